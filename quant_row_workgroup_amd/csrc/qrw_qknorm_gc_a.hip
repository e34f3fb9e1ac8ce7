// qrw_qknorm_gc_a.hip -- QK RMSNorm + RoPE kernels of chunk widths 1-4
// (granules per lane per wave); split from the other widths so the sources
// compile in parallel.
#include "qrw_qknorm.h"

namespace qrw {

void qk_run_gc1(const QkArgs& a) { qk_run<1>(a); }
void qk_run_gc2(const QkArgs& a) { qk_run<2>(a); }
void qk_run_gc3(const QkArgs& a) { qk_run<3>(a); }
void qk_run_gc4(const QkArgs& a) { qk_run<4>(a); }

}  // namespace qrw
