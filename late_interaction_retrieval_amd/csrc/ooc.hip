// ooc.hip -- out-of-core corpus scoring for gfx950 (MI355X): the corpus stays
// in host memory and is streamed to the GPU in blocks of documents, each
// block scored by the same fused forward (Flash-MaxSim Section 5
// "Out-of-Core Corpus Scaling", Table 4: peak GPU memory is set by one
// streamed block, not by the corpus).
//
// Two device buffers hold alternate blocks.  A copy stream owned by the
// library moves block k into buffer k % 2 while the caller's stream scores
// block k - 1 from the other buffer:
//   copy stream : wait(free[k%2]) -> H2D block k -> record(ready[k%2])
//   caller      : wait(ready[k%2]) -> [rebase cu] -> forward -> copy the block's
//                 scores (and argmax) into the output columns -> record(free[k%2])
// Everything is enqueued without blocking the host; the caller's stream is
// ordered after the last block.  The copy stream and the events are created
// once per device and kept for the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace maxsim {
namespace {

struct StreamState {
    hipStream_t copy = nullptr;
    hipEvent_t ready[2] = {nullptr, nullptr};
    hipEvent_t free_[2] = {nullptr, nullptr};
    std::mutex mu;  // one enqueue at a time per device (the events are shared)
    bool init = false;
};

constexpr int kMaxDevices = 64;
StreamState g_state[kMaxDevices];
std::mutex g_init_mu;

hipError_t state_for_current_device(StreamState** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    StreamState& s = g_state[dev];
    std::lock_guard<std::mutex> lk(g_init_mu);
    if (!s.init) {
        // default priority; non-blocking with respect to the null stream
        if ((e = hipStreamCreateWithFlags(&s.copy, hipStreamNonBlocking)) != hipSuccess) return e;
        for (int i = 0; i < 2; ++i) {
            if ((e = hipEventCreateWithFlags(&s.ready[i], hipEventDisableTiming)) != hipSuccess) return e;
            if ((e = hipEventCreateWithFlags(&s.free_[i], hipEventDisableTiming)) != hipSuccess) return e;
        }
        s.init = true;
    }
    *out = &s;
    return hipSuccess;
}

// out[j] = cu[b0 + j] - cu[b0], j = 0 .. nb: the block's own cu_seqlens.
__global__ __launch_bounds__(256) void rebase_cu(const int32_t* cu, int b0, int nb, int32_t* out) {
    const int base = cu[b0];
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j <= nb; j += gridDim.x * blockDim.x)
        out[j] = cu[b0 + j] - base;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t host_stream_staging_bytes(int32_t Nq, int32_t Lq, int32_t Ld, int32_t block_docs, bool with_argmax) {
    if (Nq < 1 || Lq < 1 || Ld < 1 || block_docs < 1) return 0;
    const size_t dbuf = align256((size_t)block_docs * Ld * kDim * 2);
    size_t n = 2 * dbuf + align256((size_t)Nq * block_docs * sizeof(float)) +
               align256((size_t)(block_docs + 1) * sizeof(int32_t));
    if (with_argmax) n += align256((size_t)Nq * block_docs * Lq * sizeof(int32_t));
    return n;
}

hipError_t launch_fwd_host_stream(const HostStreamArgs& a, hipStream_t stream) {
    StreamState* st = nullptr;
    hipError_t e = state_for_current_device(&st);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(st->mu);

    // staging layout: D buffer 0, D buffer 1, block scores, block cu, block argmax
    char* ws = static_cast<char*>(a.staging);
    const size_t dbuf = align256((size_t)a.block_docs * a.Ld * kDim * 2);
    char* dbufs[2] = {ws, ws + dbuf};
    float* sblk = reinterpret_cast<float*>(ws + 2 * dbuf);
    int32_t* cublk = reinterpret_cast<int32_t*>(ws + 2 * dbuf + align256((size_t)a.Nq * a.block_docs * 4));
    int32_t* ablk = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(cublk) +
                                               align256((size_t)(a.block_docs + 1) * 4));
    const bool packed = a.cu_host != nullptr;
    const char* host = static_cast<const char*>(a.D_host);

    // the staging buffers may still be read by earlier work on the caller's
    // stream: the first copy into each buffer waits for the stream's present end
    for (int i = 0; i < 2; ++i)
        if ((e = hipEventRecord(st->free_[i], stream)) != hipSuccess) return e;

    for (int b0 = 0, k = 0; b0 < a.B; b0 += a.block_docs, ++k) {
        const int nb = a.B - b0 < a.block_docs ? a.B - b0 : a.block_docs;
        const int buf = k & 1;
        int64_t r0, r1;  // host rows of the block
        if (packed) {
            r0 = a.cu_host[b0];
            r1 = a.cu_host[b0 + nb];
        } else {
            r0 = (int64_t)b0 * a.Ld;
            r1 = (int64_t)(b0 + nb) * a.Ld;
        }
        const size_t bytes = (size_t)(r1 - r0) * kDim * 2;
        if ((e = hipStreamWaitEvent(st->copy, st->free_[buf], 0)) != hipSuccess) return e;
        if (bytes > 0 &&
            (e = hipMemcpyAsync(dbufs[buf], host + r0 * kDim * 2, bytes, hipMemcpyDefault, st->copy)) != hipSuccess)
            return e;
        if ((e = hipEventRecord(st->ready[buf], st->copy)) != hipSuccess) return e;

        if ((e = hipStreamWaitEvent(stream, st->ready[buf], 0)) != hipSuccess) return e;
        FwdArgs f{};
        f.Q = a.Q;
        f.D = dbufs[buf];
        f.Nq = a.Nq;
        f.Lq = a.Lq;
        f.B = nb;
        f.Ld = a.Ld;
        f.scores = sblk;
        f.argmax = a.argmax ? ablk : nullptr;
        f.elem = a.elem;
        if (packed) {
            hipLaunchKernelGGL(rebase_cu, dim3((nb + 256) / 256), dim3(256), 0, stream, a.cu_dev, b0, nb, cublk);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            f.cu = cublk;
            f.T = r1 - r0;
            f.varlen = true;
        } else {
            f.d_lens = a.d_lens ? a.d_lens + b0 : nullptr;
            f.T = (int64_t)nb * a.Ld;  // rows of the padded block
        }
        if ((e = launch_fwd(f, stream)) != hipSuccess) return e;
        // block columns [b0, b0 + nb) of scores [Nq, B] and argmax [Nq, B, Lq]
        if ((e = hipMemcpy2DAsync(a.scores + b0, (size_t)a.B * 4, sblk, (size_t)nb * 4, (size_t)nb * 4, a.Nq,
                                  hipMemcpyDeviceToDevice, stream)) != hipSuccess)
            return e;
        if (a.argmax &&
            (e = hipMemcpy2DAsync(a.argmax + (int64_t)b0 * a.Lq, (size_t)a.B * a.Lq * 4, ablk,
                                  (size_t)nb * a.Lq * 4, (size_t)nb * a.Lq * 4, a.Nq, hipMemcpyDeviceToDevice,
                                  stream)) != hipSuccess)
            return e;
        if ((e = hipEventRecord(st->free_[buf], stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace maxsim
