// decode_noalloc.hip -- hils_decode for callers that cannot allocate device
// memory (graph capture, tight serving loops): the decode step's scratch
// (per-split partial top-K lists and partial softmax states) lives in a
// static device array of the library instead of a caller workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory:
// the device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is handed
// to the kernels.
#include <stdio.h>

#include <mutex>

#include "../../include/hils.h"
#include "hils_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[HILS_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES];  // device address of `scratch` per device (null until looked up)

}  // namespace

extern "C" hils_status_t hils_decode_noalloc(const hils_config_t *cfg, int32_t num_seqs, const void *q,
                                             const void *k_cache, const void *v_cache, const void *ksum_cache,
                                             const float *bsum_cache, const int32_t *block_table, int32_t max_pages,
                                             const int32_t *seq_lens, const void *h, const void *w_down,
                                             const void *w_up, int32_t d_model, int32_t r, void *out, float *lse,
                                             int32_t *sel_idx, hipStream_t stream) {
    char msg[256];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        snprintf(msg, sizeof(msg), "decode_noalloc: no usable current device (%d)", dev);
        return (hils_status_t)hils::report_error(HILS_ERR_HIP, msg);
    }
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) {
            snprintf(msg, sizeof(msg), "decode_noalloc: the stream belongs to device %d, current is %d", sdev,
                     dev);
            return (hils_status_t)hils::report_error(HILS_ERR_INVALID_ARG, msg);
        }
    }
    // the scratch need; 0 means the configuration is rejected, which
    // hils_decode reports below with its own message
    const size_t need = num_seqs > 0 ? hils_workspace_size(cfg, HILS_WS_DECODE, num_seqs, max_pages) : 0;
    if (need > HILS_DECODE_NOALLOC_SCRATCH_BYTES) {
        snprintf(msg, sizeof(msg),
                 "decode_noalloc: %d sequences x %d pages need %zu bytes of scratch; the static scratch holds %zu",
                 num_seqs, max_pages, need, (size_t)HILS_DECODE_NOALLOC_SCRATCH_BYTES);
        return (hils_status_t)hils::report_error(HILS_ERR_UNSUPPORTED, msg);
    }
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_scratch[dev]) {
            void *p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                snprintf(msg, sizeof(msg), "decode_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                         hipGetErrorString(e));
                return (hils_status_t)hils::report_error(HILS_ERR_HIP, msg);
            }
            g_scratch[dev] = p;
        }
        ptr = g_scratch[dev];
    }
    return hils_decode(cfg, num_seqs, q, k_cache, v_cache, ksum_cache, bsum_cache, block_table, max_pages, seq_lens,
                       h, w_down, w_up, d_model, r, out, lse, sel_idx, ptr, HILS_DECODE_NOALLOC_SCRATCH_BYTES,
                       stream);
}
