// pn_host.hpp - host-side pieces shared by the library's translation units
// (no kernels): the sampler's sizes and its host entry, and the error message
// of pn_last_error.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pn.h"

namespace pn {

constexpr int kSampleMaxK = 4096;       // largest top_k
constexpr int kSampleCap = 8192;        // candidates held in LDS
constexpr int kSampleBins = 4096;       // histogram bins per level (12 key bits)
constexpr int kSampleMaxRecent = 1024;  // tokens of a row's recent window

// Scratch of the sampler for up to `rows` rows of up to `vocab` tokens, as
// offsets in one buffer: keys [rows][vocab] u32, histogram [rows][bins] u32,
// gather counters [rows][2] u32, candidates [rows][cap] u64; 256-byte aligned.
struct SampleScratch {
    size_t keys, hist, cnt, cand, bytes;
};
constexpr size_t sample_align(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr SampleScratch sample_scratch(int rows, int vocab) {
    const size_t keys = 0;
    const size_t hist = sample_align(keys + (size_t)rows * vocab * 4);
    const size_t cnt = sample_align(hist + (size_t)rows * kSampleBins * 4);
    const size_t cand = sample_align(cnt + (size_t)rows * 2 * 4);
    return SampleScratch{keys, hist, cnt, cand, sample_align(cand + (size_t)rows * kSampleCap * 8)};
}

struct SampleScratchPtrs {
    unsigned *keys, *hist, *cnt;
    unsigned long long *cand;
};

// Check the sampling arguments of n rows over a vocabulary of V and enqueue
// the sampler on `st` with the given scratch (histogram and counters for
// rows_cap rows; `dirty`: they may not be zero, clear them first).  Returns 0
// or a PN_E* code with the message set.
int host_sample(const float *logits_dev, int n, int V, const pn_sampling_params *params, const int32_t *recent_dev,
                int n_recent, const float *u_dev, int32_t *ids_dev, const SampleScratchPtrs &sp, int rows_cap,
                bool &dirty, hipStream_t st);

// Set the message pn_last_error returns and return `code`; clear it.
int host_fail(int code, const char *fmt, ...);
void host_clear_error();

}  // namespace pn
