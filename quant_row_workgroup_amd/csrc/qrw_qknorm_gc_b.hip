// qrw_qknorm_gc_b.hip -- QK RMSNorm + RoPE kernels of chunk widths 5, 6 and 8
// (granules per lane per wave); split from the other widths so the sources
// compile in parallel.
#include "qrw_qknorm.h"

namespace qrw {

void qk_run_gc5(const QkArgs& a) { qk_run<5>(a); }
void qk_run_gc6(const QkArgs& a) { qk_run<6>(a); }
void qk_run_gc8(const QkArgs& a) { qk_run<8>(a); }

}  // namespace qrw
