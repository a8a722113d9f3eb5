// pn_noalloc.hip - pn_sample_noalloc: the sampler for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  It takes no model: its scratch is a
// file-scope device array of fixed size in this file, which each GPU the
// library runs on holds until the process ends.
//
// Host code never hands the array's name to a kernel (in host code that name
// is a host-side stand-in, not a device address): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current at
// the entry point's first call there, and kept per device.  Every call on one
// GPU shares that GPU's copy, which keeps the last call's contents; the parts
// that must start at zero (histogram, gather counters) are left zero by each
// call's last kernel and cleared by a fill kernel at a device's first call or
// after a call that stopped early.  Calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pn.h"
#include "pn_host.hpp"

using namespace pn;

namespace {

constexpr int kNoAllocRows = 16;       // rows per call
constexpr int kNoAllocVocab = 262144;  // tokens per row
constexpr SampleScratch kLayout = sample_scratch(kNoAllocRows, kNoAllocVocab);  // about 17.3 MB

__device__ __align__(256) unsigned char scratch[kLayout.bytes];

constexpr int kMaxDevices = 64;
struct Device {
    std::once_flag once;
    hipError_t err = hipSuccess;
    char *ptr = nullptr;  // this device's copy of `scratch`
    bool dirty = true;    // histogram and counters not known to be zero (first use: clear)
    std::mutex mu;        // host bookkeeping of the device's calls
};
Device g_dev[kMaxDevices];

int device_scratch(Device **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return host_fail(PN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return host_fail(PN_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    Device &d = g_dev[dev];
    std::call_once(d.once, [&d]() {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.ptr = (char *)p;
    });
    if (d.err != hipSuccess || !d.ptr)
        return host_fail(PN_EHIP, "device address of the sampler scratch on device %d: %s", dev,
                         hipGetErrorString(d.err));
    *out = &d;
    return PN_OK;
}

}  // namespace

extern "C" int pn_sample_noalloc(const float *logits_dev, int32_t n, int32_t n_vocab,
                                 const pn_sampling_params *params, const int32_t *recent_dev, int32_t n_recent,
                                 const float *u_dev, int32_t *ids_dev, void *stream) {
    host_clear_error();
    if (!logits_dev || !params || !u_dev || !ids_dev) return host_fail(PN_EINVAL, "NULL argument");
    if (n < 1 || n > kNoAllocRows) return host_fail(PN_EINVAL, "n = %d outside [1, %d]", n, kNoAllocRows);
    if (n_vocab < 1 || n_vocab > kNoAllocVocab)
        return host_fail(PN_EINVAL, "n_vocab = %d outside [1, %d]", n_vocab, kNoAllocVocab);
    Device *d = nullptr;
    if (int rc = device_scratch(&d)) return rc;
    SampleScratchPtrs sp{(unsigned *)(d->ptr + kLayout.keys), (unsigned *)(d->ptr + kLayout.hist),
                         (unsigned *)(d->ptr + kLayout.cnt), (unsigned long long *)(d->ptr + kLayout.cand)};
    std::lock_guard<std::mutex> lk(d->mu);
    return host_sample(logits_dev, n, n_vocab, params, recent_dev, n_recent, u_dev, ids_dev, sp, kNoAllocRows,
                       d->dirty, (hipStream_t)stream);
}
