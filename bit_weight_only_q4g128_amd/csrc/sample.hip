// Top-k sampling from BF16 logits (the step after the head GEMV): the
// Rumik TTS Fast Inference post samples audio tokens at temperature 0.8 with
// top-k 30 ("The Result") from the head restricted to the current codebook
// ("What Made It Faster").
//
// One workgroup per batch row:
//   1. the row's logits go to LDS as order-preserving 16-bit keys (-0 taken
//      as +0, so equal values tie);
//   2. a two-pass 8-bit radix select finds the k-th largest key T;
//   3. the keys above T are gathered, then the keys equal to T in index
//      order (a block-wide prefix count) until there are k;
//   4. one wave sorts the k entries by (logit descending, index ascending)
//      with a bitonic network over its lanes (lane exchanges in registers);
//   5. the lanes form e_i = exp(z_i - z_0), z = logit / T, their running
//      sums (a prefix scan over the lanes) and total S; the token is the
//      first entry whose running sum exceeds u * S, and p_i = e_i / S.
#include "internal.h"
#include "topk.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;

// Wave 0: the bin b (counting down from bin 255) where the running count
// first reaches k; writes b and how many of bin b are still wanted.  Lane l
// holds bins 4l .. 4l + 3; the count above its bins is the total less a
// prefix scan over the lanes (DPP), and the one lane whose bins cross k
// reports.
__device__ void find_bin(const unsigned* hist, int k, int lane, int* s_bin, int* s_need) {
    unsigned h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = hist[4 * lane + j];
    const unsigned mine = h[0] + h[1] + h[2] + h[3];
    const unsigned incl = (unsigned)wave_incl_scan_i((int)mine);   // sum over lanes <= this one
    const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
    unsigned cum = total - incl;                          // count in the bins above this lane's
#pragma unroll
    for (int j = 3; j >= 0; --j) {
        if (cum < (unsigned)k && cum + h[j] >= (unsigned)k) {
            *s_bin = 4 * lane + j;
            *s_need = k - (int)cum;
        }
        cum += h[j];
    }
}

__global__ __launch_bounds__(kThreads) void topk_sample_kernel(const uint16_t* __restrict__ logits, int V, float temperature, int k,
                                                               const float* __restrict__ u, int32_t* __restrict__ token,
                                                               int32_t* __restrict__ topk_index, float* __restrict__ topk_prob) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint16_t* keys = reinterpret_cast<uint16_t*>(lds);            // [V]
    __shared__ unsigned hist[256];
    __shared__ unsigned wsum[kThreads / 64];
    __shared__ uint32_t list[64];
    __shared__ int s_n, s_bin, s_need;

    const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t* row = logits + (size_t)m * V;
    const float um = u[m];                                        // loaded with the logits, used at the end

    // logits to LDS keys, 16 independent loads in flight per thread
    constexpr int kBatch = 16;
    for (int i0 = tid; i0 < V; i0 += kBatch * kThreads) {
        uint16_t v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = i0 + j * kThreads;
            v[j] = i < V ? row[i] : (uint16_t)0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = i0 + j * kThreads;
            if (i < V) keys[i] = (uint16_t)order_key(v[j]);
        }
    }
    hist[tid] = 0;
    if (tid == 0) s_n = 0;
    __syncthreads();

    // 2. radix select: high byte, then low byte within the chosen high byte
    for (int i = tid; i < V; i += kThreads) atomicAdd(&hist[keys[i] >> 8], 1u);
    __syncthreads();
    if (wave == 0) find_bin(hist, k, lane, &s_bin, &s_need);
    __syncthreads();
    const int hi = s_bin, need_hi = s_need;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < V; i += kThreads)
        if ((keys[i] >> 8) == hi) atomicAdd(&hist[keys[i] & 0xFF], 1u);
    __syncthreads();
    if (wave == 0) find_bin(hist, need_hi, lane, &s_bin, &s_need);
    __syncthreads();
    const uint32_t thr = ((uint32_t)hi << 8) | (uint32_t)s_bin;
    const int need_eq = s_need;                                   // entries equal to thr to take

    // 3. gather: contiguous index ranges per thread, so that equal keys can be
    // ranked in index order by a prefix count over the threads
    const int per = (V + kThreads - 1) / kThreads;
    const int i0 = tid * per, i1 = (i0 + per < V) ? i0 + per : V;
    unsigned n_eq = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t key = keys[i];
        if (key > thr) {
            const int slot = atomicAdd(&s_n, 1);
            list[slot] = (key << 16) | (0xFFFFu - (uint32_t)i);
        }
        n_eq += key == thr ? 1u : 0u;
    }
    const unsigned incl = (unsigned)wave_incl_scan_i((int)n_eq);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned rank = incl - n_eq;                                  // equal keys before this thread's range
    for (int w = 0; w < wave; ++w) rank += wsum[w];
    const int n_gt = k - need_eq;
    for (int i = i0; i < i1 && (int)rank < need_eq; ++i) {
        if (keys[i] == thr) {
            list[n_gt + rank] = (thr << 16) | (0xFFFFu - (uint32_t)i);
            ++rank;
        }
    }
    __syncthreads();

    // 4-5. sort the k entries (bitonic network over the lanes) and draw, in wave 0
    if (wave == 0)
        draw_sorted(wave_sort64<true>(lane < k ? list[lane] : 0u, lane), k, temperature, um, lane, token + m,
                      topk_index ? topk_index + (size_t)m * k : nullptr, topk_prob ? topk_prob + (size_t)m * k : nullptr);
}

// The split form for batches (a caller workspace): each batch row's logits
// are dealt to workgroups of 1024; each takes the top k of its block
// (topk.h) and publishes them, device-coherently, as candidates; the last
// block of the row to arrive at the row's counter takes the top k of all of
// them, sorts and draws.  The rows' counters sit a cache line apart.
constexpr int kSplitE2 = 8;         // candidate entries per thread in the merge (2048)

__global__ __launch_bounds__(kThreads) void topk_sample_split_kernel(const uint16_t* __restrict__ logits, int V, float temperature,
                                                                     int k, int nb, const float* __restrict__ u,
                                                                     int32_t* __restrict__ token, int32_t* __restrict__ topk_index,
                                                                     float* __restrict__ topk_prob, unsigned* cnt, uint32_t* cand,
                                                                     int M) {
    __shared__ uint32_t lists[4 * 64];
    __shared__ uint32_t scratch[4 * 64 * kSplitE2];
    __shared__ unsigned s_prev;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = blockIdx.x / nb, j = blockIdx.x - m * nb;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(logits + (size_t)m * V, (uint32_t)V * 2u);
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = j * kSplitBlock + tid + 256 * i;
        v[i] = __builtin_amdgcn_raw_buffer_load_b16(rl, (int)(col < V ? col * 2 : 0x7FFFFFF0), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = j * kSplitBlock + tid + 256 * i;
        v[i] = topk_entry(v[i], col) & (col < V ? 0xFFFFFFFFu : 0u);
    }
    uint32_t top = wg_topk<4>(v, k, lists, scratch, wave, lane);
    const int nc = nb * k;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cand, (uint32_t)(M * nc * 4));
    if (nb > 1) {
        if (wave == 0 && lane < k)
            __builtin_amdgcn_raw_buffer_store_b32(top, rc, (m * nc + j * k + lane) * 4, 0, 16);
        if (!arrive_last(cnt + (size_t)m * kCtrWords, nb, tid, &s_prev)) return;
        uint32_t w[kSplitE2];
#pragma unroll
        for (int i = 0; i < kSplitE2; ++i) {
            const int c = tid + 256 * i;
            w[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(c < nc ? (m * nc + c) * 4 : 0x7FFFFFF0), 0, 16);
        }
        top = wg_topk<kSplitE2>(w, k, lists, scratch, wave, lane);
    }
    if (wave == 0)
        draw_sorted(top, k, temperature, u[m], lane, token + m, topk_index ? topk_index + (size_t)m * k : nullptr,
                    topk_prob ? topk_prob + (size_t)m * k : nullptr);
}

}  // namespace

size_t topk_sample_split_ws_bytes(int M, int V, int top_k) {
    const int nb = (V + kSplitBlock - 1) / kSplitBlock;
    if (nb * top_k > 256 * kSplitE2) return 0;
    const size_t counters = (size_t)M * kCtrStride;
    return counters + (nb > 1 ? (size_t)M * nb * top_k * 4 : 0);
}

hipError_t launch_topk_sample_split(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u,
                                    int32_t* token, int32_t* topk_index, float* topk_prob, void* ws, hipStream_t s) {
    const int nb = (V + kSplitBlock - 1) / kSplitBlock;
    unsigned* cnt = static_cast<unsigned*>(ws);
    uint32_t* cand = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + (size_t)M * kCtrStride);
    return launch_kernel(topk_sample_split_kernel, dim3(M * nb), dim3(kThreads), 0, s, logits, V, temperature, top_k, nb, u, token,
                         topk_index, topk_prob, cnt, cand, M);
}

hipError_t launch_topk_sample(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u, int32_t* token,
                              int32_t* topk_index, float* topk_prob, hipStream_t s) {
    return launch_kernel(topk_sample_kernel, dim3(M), dim3(kThreads), (size_t)V * 2, s, logits, V, temperature, top_k, u, token,
                         topk_index, topk_prob);
}

}  // namespace q4
