// Instantiations of the varlen prefill kernel: head dim 128, GQA groups of 3, 5, 6, 7, 16 and 32.

#include "prefill_launch.h"

namespace pa {

int prefill_dispatch_k128_odd(PA_PREFILL_DISPATCH_ARGS) {
    switch (G) {
        PA_PREFILL_CASE(128, 3)
        PA_PREFILL_CASE(128, 5)
        PA_PREFILL_CASE(128, 6)
        PA_PREFILL_CASE(128, 7)
        PA_PREFILL_CASE(128, 16)
        PA_PREFILL_CASE(128, 32)
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace pa
