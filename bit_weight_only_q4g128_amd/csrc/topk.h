// Top-k selection and the draw over BF16 logits, shared by the sampler and
// the head GEMV with fused sampling.  The Rumik TTS Fast Inference post
// samples every audio token at temperature 0.8 with top-k 30 ("The Result")
// from the head restricted to the current codebook ("What Made It Faster").
//
// An entry packs one logit and its index as key << 16 | (0xFFFF - index),
// where key is an order-preserving 16-bit image of the BF16 logit (-0 taken
// as +0).  Entries of distinct indices are distinct, and entry order is the
// sampling order: larger logit first, then lower index.  0 is never an entry
// (it would be a NaN logit) and pads.
#pragma once

#include "common.h"

namespace q4 {

__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
    if (bits == 0x8000u) bits = 0;                      // -0 ties with +0
    return (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
    const uint32_t bits = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
    return __builtin_bit_cast(float, bits << 16);
}
__device__ __forceinline__ uint32_t topk_entry(uint32_t logit_bits, int index) {
    return (order_key(logit_bits) << 16) | (0xFFFFu - (uint32_t)index);
}

// The k-th largest of a wave's entries (E per lane), built bit by bit from
// the top: the largest T with at least k entries >= T.  With distinct
// nonzero entries, at least k of them, exactly k entries are >= T.  The
// counts are ballots, so the search is wave-uniform with no LDS traffic.
template <int E>
__device__ __forceinline__ uint32_t wave_kth(const uint32_t (&v)[E], int k) {
    uint32_t t = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        int n = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) n += __popcll(__ballot(v[j] >= c));
        if (n >= k) t = c;
    }
    return t;
}

// Inclusive prefix sum of an integer over the 64 lanes (DPP: shifts within
// rows of 16, then the row totals broadcast forward).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
    x += dpp_i<0x111>(x);        // row_shr:1
    x += dpp_i<0x112>(x);        // row_shr:2
    x += dpp_i<0x114>(x);        // row_shr:4
    x += dpp_i<0x118>(x);        // row_shr:8
    x += dpp_i<0x142, 0xA>(x);   // row_bcast:15 into rows 1, 3
    x += dpp_i<0x143, 0xC>(x);   // row_bcast:31 into rows 2, 3
    return x;
}

// Writes the wave's nonzero entries >= T to list[0 ..) (lane by lane, each
// lane's in register order) and returns how many there were: per-lane
// counts, one prefix scan over the lanes for the offsets.
template <int E>
__device__ __forceinline__ int wave_take(const uint32_t (&v)[E], uint32_t T, uint32_t* list) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) c += (v[j] >= T && v[j] != 0u) ? 1 : 0;
    const int incl = wave_incl_scan_i(c);
    int pos = incl - c;
#pragma unroll
    for (int j = 0; j < E; ++j)
        if (v[j] >= T && v[j] != 0u) list[pos++] = v[j];
    return __builtin_amdgcn_readlane(incl, 63);
}

// The 64 lanes' values sorted descending across the lanes (bitonic network).
__device__ __forceinline__ uint32_t wave_sort64_desc(uint32_t v, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t o = __shfl_xor(v, stride);
            const bool up = ((lane & size) == 0);            // this half of the sequence descends
            const bool lower = (lane & stride) == 0;
            const bool keep_max = (up == lower);
            v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
        }
    }
    return v;
}

// The top k (1 <= k <= 64) of a wave's entries (E per lane, distinct where
// nonzero), sorted descending in lanes 0 .. k-1 (fewer nonzero entries: all
// of them, then zeros).  The k-th largest lane maximum L is a lower bound of
// the k-th largest entry (k lanes hold an entry >= L), so the entries >= L --
// at least k, at most k * E, usually few more than k -- are the candidates:
// up to 64 of them are sorted directly; more take the bit-by-bit threshold
// first.  scratch: 64 E words of LDS, private to the wave.
template <int E>
__device__ uint32_t wave_topk_sorted(const uint32_t (&v)[E], int k, uint32_t* scratch, int lane) {
    uint32_t mx = v[0];
#pragma unroll
    for (int j = 1; j < E; ++j) mx = v[j] > mx ? v[j] : mx;
    const uint32_t L = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort64_desc(mx, lane), k - 1);
    const int n = wave_take<E>(v, L, scratch);
    __builtin_amdgcn_wave_barrier();
    if (n <= 64) return wave_sort64_desc(lane < n ? scratch[lane] : 0u, lane);
    uint32_t w[E];
#pragma unroll
    for (int j = 0; j < E; ++j) w[j] = lane + 64 * j < n ? scratch[lane + 64 * j] : 0u;
    __builtin_amdgcn_wave_barrier();
    const uint32_t T = wave_kth<E>(w, k);
    const int m = wave_take<E>(w, T, scratch);
    __builtin_amdgcn_wave_barrier();
    return wave_sort64_desc(lane < m ? scratch[lane] : 0u, lane);
}

// The top 64 of two lists sorted descending across the lanes, sorted:
// max(x_i, y_63-i) holds them as a bitonic sequence, which a bitonic merge
// sorts.
__device__ __forceinline__ uint32_t merge_top64(uint32_t x, uint32_t y, int lane) {
    const uint32_t yr = __shfl(y, 63 - lane);
    uint32_t v = x > yr ? x : yr;
#pragma unroll
    for (int stride = 32; stride > 0; stride >>= 1) {
        const uint32_t o = __shfl_xor(v, stride);
        v = (lane & stride) == 0 ? (v > o ? v : o) : (v < o ? v : o);
    }
    return v;
}

// Top k (1 <= k <= 64) of the entries of a 256-thread workgroup (E per
// thread, distinct where nonzero, at least k nonzero): each wave takes its own
// top k, sorted; wave 0 merges the four lists.  Returns, in wave 0, the top k
// sorted descending in lanes 0 .. k-1 (0 elsewhere).  LDS: lists holds
// 4 x 64 words, scratch 4 x 64 E words.  Every thread must call.
template <int E>
__device__ uint32_t wg_topk(const uint32_t (&v)[E], int k, uint32_t* lists, uint32_t* scratch, int wave, int lane) {
    const uint32_t r = wave_topk_sorted<E>(v, k, scratch + 64 * E * wave, lane);
    lists[64 * wave + lane] = lane < k ? r : 0u;
    __syncthreads();
    uint32_t top = 0u;
    if (wave == 0) {
        const uint32_t ab = merge_top64(lists[lane], lists[64 + lane], lane);
        const uint32_t cd = merge_top64(lists[128 + lane], lists[192 + lane], lane);
        top = merge_top64(ab, cd, lane);
        top = lane < k ? top : 0u;
    }
    __syncthreads();
    return top;
}

// Hand-over between the workgroups of one launch: this workgroup's
// device-coherent (sc1) stores are acknowledged (vmcnt(0): the coherence
// point has accepted them), the workgroup's threads meet, and one relaxed
// agent-scope atomic arrives at counter c; true in the last of n arrivals,
// which also resets c.  The last arriver then reads the others' data with sc1
// loads, issued after its atomic returned.  Counters of different hand-overs
// sit on different cache lines (atomics on one line serialize).
__device__ __forceinline__ bool arrive_last(unsigned* c, int n, int tid, unsigned* s_prev) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) *s_prev = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool last = *s_prev == (unsigned)(n - 1);
    if (last && tid == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
    return last;
}

// Inclusive prefix sum over the 64 lanes (DPP: shifts within rows of 16,
// then the row totals broadcast forward).
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += dpp<0x111>(x);        // row_shr:1
    x += dpp<0x112>(x);        // row_shr:2
    x += dpp<0x114>(x);        // row_shr:4
    x += dpp<0x118>(x);        // row_shr:8
    x += dpp<0x142, 0xA>(x);   // row_bcast:15 into rows 1, 3
    x += dpp<0x143, 0xC>(x);   // row_bcast:31 into rows 2, 3
    return x;
}

// Wave-wide (all 64 lanes) draw for one batch row: lanes 0 .. k-1 hold the
// top k entries sorted descending.  With z = logit / T the lanes form
// e_i = exp(z_i - z_0); S is their sum and c_i the running sums (a prefix
// scan over the lanes); the token is the first entry whose running sum
// exceeds u * S (the last if none does), and p_i = e_i / S.
__device__ __forceinline__ void draw_sorted(uint32_t v, int k, float temperature, float um, int lane, int32_t* token,
                                            int32_t* topk_index, float* topk_prob) {
    const float z = key_value(v >> 16) / temperature;
    const float z0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, z)));
    const float e = lane < k ? expf(z - z0) : 0.f;
    const float c = wave_incl_scan(e);
    const float S = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 63));
    const unsigned long long over = __ballot(c > um * S && lane < k - 1);
    const int pick = over ? (int)__builtin_ctzll(over) : k - 1;
    const int index = (int)(0xFFFFu - (v & 0xFFFFu));
    if (lane == pick) *token = index;
    if (lane < k) {
        if (topk_index) topk_index[lane] = index;
        if (topk_prob) topk_prob[lane] = e / S;
    }
}

}  // namespace q4
