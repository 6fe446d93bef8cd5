// One table of recurrence kernels of the gated delta rule library: state
// storage type GDR_ST (uint16_t = bf16 bits, or float) and kernel mode
// GDR_MODE (kPlain 0, kVerify 1, kSnap 2, plus kBetaCols 4), both set on the
// compiler command line.  The library links ten of these objects.
#include "gdr_device.h"

#if !defined(GDR_ST) || !defined(GDR_MODE)
#error "gdr_rec_table.hip is compiled with -DGDR_ST=<type> -DGDR_MODE=<mode>"
#endif

namespace gdr {
template hipError_t launch_rec_table<GDR_ST, GDR_MODE>(const RecParams&, const LaunchShape&,
                                                       hipStream_t);
}  // namespace gdr
