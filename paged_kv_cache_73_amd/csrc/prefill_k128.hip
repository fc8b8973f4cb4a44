// Instantiations of the varlen prefill kernel: head dim 128, GQA groups of 1, 2, 4 and 8.

#include "prefill_launch.h"

namespace pa {

int prefill_dispatch_k128(PA_PREFILL_DISPATCH_ARGS) {
    switch (G) {
        PA_PREFILL_CASE(128, 1)
        PA_PREFILL_CASE(128, 2)
        PA_PREFILL_CASE(128, 4)
        PA_PREFILL_CASE(128, 8)
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace pa
