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

// Compare-exchange partners of a bitonic network over the 64 lanes, with no
// LDS traffic: the larger and the smaller of the values of lanes l and
// l ^ S.  S = 1, 2: quad permutes; 4: row shifts with bank masks; 8: a row
// rotation; 16, 32: the permlane swaps, whose two results hold, at every
// lane, its own value and its partner's (in either order).
template <int S>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t& hi, uint32_t& lo) {
    uint32_t a = v, b;
    if constexpr (S == 1) {
        b = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);    // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        b = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);    // quad_perm [2,3,0,1]
    } else if constexpr (S == 4) {
        const int t = __builtin_amdgcn_update_dpp((int)v, (int)v, 0x104, 0xF, 0x5, false);  // row_shl:4 into lanes 0-3, 8-11
        b = (uint32_t)__builtin_amdgcn_update_dpp(t, (int)v, 0x114, 0xF, 0xA, false);       // row_shr:4 into lanes 4-7, 12-15
    } else if constexpr (S == 8) {
        b = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);   // row_ror:8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = r[0];
        b = r[1];
    } else {
        static_assert(S == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = r[0];
        b = r[1];
    }
    hi = a > b ? a : b;
    lo = a > b ? b : a;
}

// One compare-exchange step at distance S: lane l keeps the larger value
// when keep_max.
template <int S>
__device__ __forceinline__ uint32_t cx(uint32_t v, bool keep_max) {
    uint32_t hi, lo;
    lane_pair<S>(v, hi, lo);
    return keep_max ? hi : lo;
}

// Step (SIZE, S) of the bitonic sort: blocks of SIZE lanes alternate
// between descending and ascending (the last, SIZE = 64, in the sort's
// direction), and within one the lower lane of each pair keeps the value
// that comes first.
template <bool DESC, int SIZE, int S>
__device__ __forceinline__ uint32_t sort_step(uint32_t v, int lane) {
    const bool first_desc = ((lane & SIZE) == 0) == DESC;   // (SIZE = 64: true for every lane when DESC)
    return cx<S>(v, first_desc == ((lane & S) == 0));
}

// The 64 lanes' values sorted across the lanes, descending (DESC) or
// ascending: the bitonic network, 21 steps.
template <bool DESC>
__device__ __forceinline__ uint32_t wave_sort64(uint32_t v, int lane) {
    v = sort_step<DESC, 2, 1>(v, lane);
    v = sort_step<DESC, 4, 2>(v, lane);
    v = sort_step<DESC, 4, 1>(v, lane);
    v = sort_step<DESC, 8, 4>(v, lane);
    v = sort_step<DESC, 8, 2>(v, lane);
    v = sort_step<DESC, 8, 1>(v, lane);
    v = sort_step<DESC, 16, 8>(v, lane);
    v = sort_step<DESC, 16, 4>(v, lane);
    v = sort_step<DESC, 16, 2>(v, lane);
    v = sort_step<DESC, 16, 1>(v, lane);
    v = sort_step<DESC, 32, 16>(v, lane);
    v = sort_step<DESC, 32, 8>(v, lane);
    v = sort_step<DESC, 32, 4>(v, lane);
    v = sort_step<DESC, 32, 2>(v, lane);
    v = sort_step<DESC, 32, 1>(v, lane);
    v = sort_step<DESC, 64, 32>(v, lane);
    v = sort_step<DESC, 64, 16>(v, lane);
    v = sort_step<DESC, 64, 8>(v, lane);
    v = sort_step<DESC, 64, 4>(v, lane);
    v = sort_step<DESC, 64, 2>(v, lane);
    v = sort_step<DESC, 64, 1>(v, lane);
    return v;
}

// The top 64 of two lists sorted across the lanes, x descending and y
// ascending, sorted: max(x_l, y_l) holds them as a bitonic sequence, which
// a bitonic merge (6 steps) sorts.
template <bool DESC>
__device__ __forceinline__ uint32_t merge_top64(uint32_t x, uint32_t y, int lane) {
    uint32_t v = x > y ? x : y;
    v = cx<32>(v, ((lane & 32) == 0) == DESC);
    v = cx<16>(v, ((lane & 16) == 0) == DESC);
    v = cx<8>(v, ((lane & 8) == 0) == DESC);
    v = cx<4>(v, ((lane & 4) == 0) == DESC);
    v = cx<2>(v, ((lane & 2) == 0) == DESC);
    v = cx<1>(v, ((lane & 1) == 0) == DESC);
    return v;
}

// The candidates for the top k (1 <= k <= 64) of a wave's entries (E per
// lane, distinct where nonzero), sorted across the lanes: at most 64 entries
// that include the k largest (all nonzero entries when there are fewer),
// descending from lane 0 or ascending up to lane 63, zeros in the other
// lanes.  The k-th largest lane maximum L is a lower bound of the k-th
// largest entry (k lanes hold an entry >= L), so the entries >= L -- at
// least k, at most k * E, usually few more than k -- are the candidates: up
// to 64 of them are sorted directly; more are first cut to exactly the k
// largest by the bit-by-bit threshold.  scratch: 64 E words of LDS, private
// to the wave.
template <int E, bool DESC>
__device__ uint32_t wave_topk_sorted(const uint32_t (&v)[E], int k, uint32_t* scratch, int lane) {
    uint32_t mx = v[0];
#pragma unroll
    for (int j = 1; j < E; ++j) mx = v[j] > mx ? v[j] : mx;
    const uint32_t L = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort64<true>(mx, lane), k - 1);
    int n = wave_take<E>(v, L, scratch);
    __builtin_amdgcn_wave_barrier();
    if (n > 64) {
        uint32_t w[E];
#pragma unroll
        for (int j = 0; j < E; ++j) w[j] = lane + 64 * j < n ? scratch[lane + 64 * j] : 0u;
        __builtin_amdgcn_wave_barrier();
        n = wave_take<E>(w, wave_kth<E>(w, k), scratch);
        __builtin_amdgcn_wave_barrier();
    }
    return wave_sort64<DESC>(lane < n ? scratch[lane] : 0u, lane);
}

// Top k (1 <= k <= 64) of the entries of a 256-thread workgroup (E per
// thread, distinct where nonzero, at least k nonzero): each wave sorts its
// own candidates (waves 0 and 2 descending, 1 and 3 ascending), and wave 0
// merges the four lists (a descending and an ascending list merge in one
// step, so no list is reversed).  Returns, in wave 0, the top k sorted descending in lanes
// 0 .. k-1 (0 elsewhere).  LDS: lists holds 4 x 64 words, scratch 4 x 64 E
// words.  Every thread must call.
template <int E>
__device__ uint32_t wg_topk(const uint32_t (&v)[E], int k, uint32_t* lists, uint32_t* scratch, int wave, int lane) {
    uint32_t* ws = scratch + 64 * E * wave;
    lists[64 * wave + lane] = (wave & 1) ? wave_topk_sorted<E, false>(v, k, ws, lane) : wave_topk_sorted<E, true>(v, k, ws, lane);
    __syncthreads();
    uint32_t top = 0u;
    if (wave == 0) {
        const uint32_t ab = merge_top64<true>(lists[lane], lists[64 + lane], lane);
        const uint32_t cd = merge_top64<false>(lists[128 + lane], lists[192 + lane], lane);
        top = merge_top64<true>(ab, cd, lane);
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
