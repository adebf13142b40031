// Born-rule attention forward on bf16 planes at head width 128 (16-query
// tiles, 16 x 16 x 32 bf16 products): the kernel of born_bf16_q16_impl.h at
// this width.
#define Q16_D 128
#include "born_bf16_q16_impl.h"
