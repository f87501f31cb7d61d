// prefill_b8.hip -- the large-M kernel instantiated for 8-bit integer codes
// (its own translation unit so the code widths compile in parallel).
#include "prefill.h"

namespace w4a16 {

template void launch_intb_prefill<8>(W4A16_PREFILL_ARGS);

}  // namespace w4a16
