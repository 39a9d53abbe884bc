// msa_prof_off.cpp — the launch hooks of the product library: they do nothing
// and hold no state. The measurement build links msa_timing.cpp instead.
#include "msa_internal.hpp"

namespace msa {
void prof_before(int, hipStream_t) {}
void prof_after(int, hipStream_t) {}
}  // namespace msa
