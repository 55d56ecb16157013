// Stream kernel instantiations for f32 inputs (one translation unit per
// input type so the kernel variants compile in parallel).
#include "stream.h"

namespace tlg {
template int launch_stream_in<TLG_F32>(const tlg_plan&, const void*, const void*, const void*, void*, void*,
                                        hipStream_t);
}  // namespace tlg
