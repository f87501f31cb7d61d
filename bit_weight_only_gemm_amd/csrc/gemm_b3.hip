// gemm_b3.hip -- the decode kernel instantiated for 3-bit integer codes (its
// own translation unit so the code widths compile in parallel).
#include "decode.h"

namespace w4a16 {

template void launch_intb_decode<3>(int, bool, int, int, int, const DecodeArgs&);

}  // namespace w4a16
