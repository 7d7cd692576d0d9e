// Generation tags of the single-read LayerNorm kernel's exchange words.
//
// A workgroup of ln_single_ctl_kernel publishes its moments of a sample as
// two fp64 words whose lowest 8 mantissa bits are replaced by a tag derived
// from the launch's generation (the count of control-wave launches on the
// workspace).  An aligned 8-byte store is seen whole or not at all, so a
// reader that finds the current tag in both words has this launch's values,
// without a separate flag.  Clearing the tag changes a value by at most
// 2^-44 relative, the same in every launch.
//
// The generation is kept in [0, 255) (it advances as (g + 1) mod 255, so no
// counter wrap ever makes two consecutive launches share a tag) and the tag
// is 1 + generation, never 0.  The words live in a region of the workspace
// that only control-wave launches write, besides the zeroing kernel, whose
// 0 no tag matches (nor would an element count, an integer below 2^44 as a
// double, whose low 8 mantissa bits are 0, as the other schedules store in
// their own slots).  Consecutive generations have different tags, and a
// control-wave launch writes every word it reads (a shape always runs the
// same tile), so the only words a reader can find are the current launch's,
// the previous control-wave launch's, or words no tag matches.
//
// Host and device versions are the same code (a CPU test checks them).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace normfwd {

__host__ __device__ inline uint32_t ln_next_generation(uint32_t generation) { return (generation + 1u) % 255u; }
__host__ __device__ inline uint32_t ln_tag_of(uint32_t generation) { return 1u + generation % 255u; }

__host__ __device__ inline uint64_t ln_bits(double v) { return __builtin_bit_cast(uint64_t, v); }
__host__ __device__ inline double ln_from_bits(uint64_t b) { return __builtin_bit_cast(double, b); }

__host__ __device__ inline double ln_tag_word(double v, uint32_t tag)
{
    return ln_from_bits((ln_bits(v) & ~(uint64_t)0xFF) | (uint64_t)(tag & 0xFFu));
}
__host__ __device__ inline bool ln_has_tag(double v, uint32_t tag)
{
    return (ln_bits(v) & (uint64_t)0xFF) == (uint64_t)(tag & 0xFFu);
}
__host__ __device__ inline double ln_untag(double v) { return ln_from_bits(ln_bits(v) & ~(uint64_t)0xFF); }

}  // namespace normfwd
