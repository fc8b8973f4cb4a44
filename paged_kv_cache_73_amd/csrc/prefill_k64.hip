// Instantiations of the varlen prefill kernel: head dim 64, every GQA group.

#include "prefill_launch.h"

namespace pa {

int prefill_dispatch_k64(PA_PREFILL_DISPATCH_ARGS) {
    switch (G) {
        PA_PREFILL_CASE(64, 1)
        PA_PREFILL_CASE(64, 2)
        PA_PREFILL_CASE(64, 3)
        PA_PREFILL_CASE(64, 4)
        PA_PREFILL_CASE(64, 5)
        PA_PREFILL_CASE(64, 6)
        PA_PREFILL_CASE(64, 7)
        PA_PREFILL_CASE(64, 8)
        PA_PREFILL_CASE(64, 16)
        PA_PREFILL_CASE(64, 32)
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace pa
