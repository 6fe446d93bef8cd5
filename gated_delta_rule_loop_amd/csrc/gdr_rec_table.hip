// One table of recurrence kernels of the gated delta rule library: per-token
// work type GDR_WT and state storage type GDR_ST (each uint16_t = bf16 bits,
// or float) and kernel mode GDR_MODE (kPlain 0, kVerify 1, kSnap 2, plus
// kBetaCols 4), all set on the compiler command line.  The library links
// twenty of these objects.
#include "gdr_device.h"

#if !defined(GDR_WT) || !defined(GDR_ST) || !defined(GDR_MODE)
#error "gdr_rec_table.hip is compiled with -DGDR_WT=<type> -DGDR_ST=<type> -DGDR_MODE=<mode>"
#endif

namespace gdr {
template hipError_t launch_rec_table<GDR_WT, GDR_ST, GDR_MODE>(const RecParams&,
                                                               const LaunchShape&, hipStream_t);
}  // namespace gdr
