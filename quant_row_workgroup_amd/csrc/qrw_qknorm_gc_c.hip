// qrw_qknorm_gc_c.hip -- QK RMSNorm + RoPE kernels of chunk widths 10 and 12
// (granules per lane per wave); split from the other widths so the sources
// compile in parallel.
#include "qrw_qknorm.h"

namespace qrw {

void qk_run_gc10(const QkArgs& a) { qk_run<10>(a); }
void qk_run_gc12(const QkArgs& a) { qk_run<12>(a); }

}  // namespace qrw
