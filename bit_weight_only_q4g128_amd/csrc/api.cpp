// C ABI of libq4gemv.so: host-side argument checks and kernel selection.
// Declarations and the contract live in include/q4gemv.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4gemv.h"
#include "internal.h"

using q4::Fmt;
using q4::GemvArgs;

namespace {

constexpr int kMaxM = 64;
static_assert(Q4GEMV_NOALLOC_SCRATCH_BYTES == q4::kNoAllocScratchBytes, "header and library disagree on the built-in scratch");
constexpr long kMaxK = 32768;
constexpr long kMaxN = 1L << 24;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_common(const void* x, int M, int K, int N, const void* y) {
    if (!x || !y) return Q4_EINVAL_PTR;
    if (M < 1 || M > kMaxM || N < 1 || N > kMaxN || K < 1 || K > kMaxK) return Q4_EINVAL_SHAPE;
    if (!aligned(x, 16) || !aligned(y, 2)) return Q4_EALIGN;
    return Q4_OK;
}

bool variant_ok(int variant) {
    return variant == Q4_VARIANT_AUTO || variant == Q4_VARIANT_DOT2 || variant == Q4_VARIANT_MFMA || variant == Q4_VARIANT_STREAM ||
           variant == Q4_VARIANT_TILED || variant == Q4_VARIANT_SKINNY;
}

// Kernel choice for Q4_VARIANT_AUTO.  Small batches on rows of 1-4 KB go to
// the streaming kernel, other small batches to the packed-dot kernel; larger
// batches to the tiled matrix-core kernel where K allows it (K % 128 == 0 and
// the int4 group parameters fit LDS, or a split), else to the per-task
// matrix-core kernel.  `split`: a workspace allows K splits.  Without one,
// NVFP4 and BF16 matrices take the tiled kernel only when their 64-row blocks
// alone fill the GPU (N >= 16384): with fewer rows the per-task kernel, which
// splits K inside its workgroups, is faster for these formats (measured).
constexpr int kTiledRowsAlone = 64 * 256;
// Prefill above 64 batch rows: the large-tile GEMM kernel once its
// 128 x 128 tiles number at least this many (one per CU), else the tiled
// decode kernel over batch chunks, whose 64-row blocks occupy more CUs.
constexpr long kGemmMinTiles = 256;
int pick(Fmt fmt, int variant, int M, int N, int K, bool split = false) {
    if (variant == Q4_VARIANT_DOT2) return q4::dot2_supported(fmt, K) ? Q4_VARIANT_DOT2 : -1;
    if (variant == Q4_VARIANT_MFMA) return Q4_VARIANT_MFMA;
    if (variant == Q4_VARIANT_STREAM) return q4::stream_supported(fmt, M, K) ? Q4_VARIANT_STREAM : -1;
    if (variant == Q4_VARIANT_TILED) return q4::mm_supported(fmt, M, K, split) ? Q4_VARIANT_TILED : -1;
    if (variant == Q4_VARIANT_SKINNY) return q4::skinny_supported(fmt, M, K, split) ? Q4_VARIANT_SKINNY : -1;
    if (M <= 4 && q4::stream_supported(fmt, M, K)) return Q4_VARIANT_STREAM;
    if (M <= 4 && q4::dot2_supported(fmt, K)) return Q4_VARIANT_DOT2;
    if (q4::skinny_supported(fmt, M, K, split)) return Q4_VARIANT_SKINNY;
    if (q4::mm_supported(fmt, M, K, split) && (fmt == q4::kFmtQ4 || split || N >= kTiledRowsAlone)) return Q4_VARIANT_TILED;
    return Q4_VARIANT_MFMA;
}

int run(Fmt fmt, int chosen, const GemvArgs* a, int count, void* stream, void* ws = nullptr, size_t ws_bytes = 0) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (chosen) {
        case Q4_VARIANT_DOT2: e = q4::launch_dot2(fmt, a, count, s); break;
        case Q4_VARIANT_STREAM: e = q4::launch_stream(fmt, a, count, s); break;
        case Q4_VARIANT_TILED: e = q4::launch_mm(fmt, a, count, ws, ws_bytes, s); break;
        case Q4_VARIANT_SKINNY: {
            Fmt f[q4::kMaxTasks];
            for (int i = 0; i < count; ++i) f[i] = fmt;
            e = q4::launch_skinny(f, a, count, ws, ws_bytes, s);
            break;
        }
        default: e = q4::launch_mfma(fmt, a, count, s); break;
    }
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

int run(Fmt fmt, int chosen, const GemvArgs& a, void* stream) { return run(fmt, chosen, &a, 1, stream); }

// Validation of one int4 task; fills `a` and the input ranges.
int check_q4(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N,
             uint16_t* y, GemvArgs& a, Range in[4], Range& out) {
    int rc = check_common(x, M, K, N, y);
    if (rc) return rc;
    if (!qweight || !scale || !minv) return Q4_EINVAL_PTR;
    if (K % 128) return Q4_EINVAL_SHAPE;
    if (!aligned(qweight, 16) || !aligned(scale, 2) || !aligned(minv, 2)) return Q4_EALIGN;
    const size_t G = (size_t)K / 128;
    in[0] = range_of(x, (size_t)M * K * 2);
    in[1] = range_of(qweight, (size_t)N * K / 2);
    in[2] = range_of(scale, (size_t)N * G * 2);
    in[3] = range_of(minv, (size_t)N * G * 2);
    out = range_of(y, (size_t)M * N * 2);
    a = GemvArgs{};
    a.x = x; a.w = qweight; a.scale = scale; a.minv = minv; a.y = y; a.M = M; a.N = N; a.K = K;
    return Q4_OK;
}

// Validation of one NVFP4 task.
int check_nv(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale, int N,
             uint16_t* y, GemvArgs& a, Range in[4], Range& out) {
    int rc = check_common(x, M, K, N, y);
    if (rc) return rc;
    if (!qweight || !scale_e4m3) return Q4_EINVAL_PTR;
    if (K % 32) return Q4_EINVAL_SHAPE;
    if (!aligned(qweight, 16)) return Q4_EALIGN;
    in[0] = range_of(x, (size_t)M * K * 2);
    in[1] = range_of(qweight, (size_t)N * K / 2);
    in[2] = range_of(scale_e4m3, (size_t)N * K / 16);
    in[3] = Range{0, 0};
    out = range_of(y, (size_t)M * N * 2);
    a = GemvArgs{};
    a.x = x; a.w = qweight; a.scale8 = scale_e4m3; a.gscale = global_scale; a.y = y; a.M = M; a.N = N; a.K = K;
    return Q4_OK;
}

// Validation of one BF16 task.
int check_bf(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* y, GemvArgs& a, Range in[4], Range& out) {
    int rc = check_common(x, M, K, N, y);
    if (rc) return rc;
    if (!w) return Q4_EINVAL_PTR;
    if (K % 8) return Q4_EINVAL_SHAPE;
    if (!aligned(w, 16)) return Q4_EALIGN;
    in[0] = range_of(x, (size_t)M * K * 2);
    in[1] = range_of(w, (size_t)N * K * 2);
    in[2] = in[3] = Range{0, 0};
    out = range_of(y, (size_t)M * N * 2);
    a = GemvArgs{};
    a.x = x; a.w = reinterpret_cast<const uint8_t*>(w); a.y = y; a.M = M; a.N = N; a.K = K;
    return Q4_OK;
}

// Kernel family for a validated group of one format: the matrix cores if any
// task needs them (the tiled kernel if every task can use it), the streaming
// kernel if every task can use it, else the packed-dot kernel (or the matrix
// cores where that cannot run); then the alias checks across tasks.
int plan_checked(Fmt fmt, const GemvArgs* a, const Range (*in)[4], const Range* out, int count, int M, int variant, bool split,
                 int* chosen_out) {
    int n_big = 0, n_tiled = 0, n_stream = 0, n_skinny = 0, n_tiled_ok = 0;
    for (int i = 0; i < count; ++i) {
        const int c = pick(fmt, variant, M, a[i].N, a[i].K, split);
        if (c < 0) return Q4_EVARIANT;
        n_big += c == Q4_VARIANT_MFMA || c == Q4_VARIANT_TILED || c == Q4_VARIANT_SKINNY;
        n_tiled += c == Q4_VARIANT_TILED;
        n_stream += c == Q4_VARIANT_STREAM;
        n_skinny += c == Q4_VARIANT_SKINNY;
        n_tiled_ok += q4::mm_supported(fmt, M, a[i].K, split);
    }
    int chosen;
    if (n_skinny == count) chosen = Q4_VARIANT_SKINNY;
    else if (n_big) chosen = (n_tiled + n_skinny == count && n_tiled_ok == count) ? Q4_VARIANT_TILED : Q4_VARIANT_MFMA;
    else chosen = n_stream == count ? Q4_VARIANT_STREAM : Q4_VARIANT_DOT2;
    if (chosen == Q4_VARIANT_DOT2) {
        for (int i = 0; i < count; ++i)
            if (!q4::dot2_supported(fmt, a[i].K)) chosen = Q4_VARIANT_MFMA;
    }
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            for (int r = 0; r < 4; ++r)
                if (overlaps(out[i], in[j][r])) return Q4_EALIAS;
            if (i != j && overlaps(out[i], out[j])) return Q4_EALIAS;
        }
    *chosen_out = chosen;
    return Q4_OK;
}

// Workspace a planned grouped launch can use (0: no K split planned).
size_t grouped_ws_bytes(Fmt fmt, int chosen, const GemvArgs* a, int count) {
    if (chosen == Q4_VARIANT_TILED) return q4::mm_workspace_bytes(fmt, a, count);
    if (chosen == Q4_VARIANT_SKINNY) {
        Fmt f[q4::kMaxTasks];
        for (int i = 0; i < count; ++i) f[i] = fmt;
        return q4::skinny_workspace_bytes(f, a, count);
    }
    return 0;
}

// A grouped call of one format after validation: a workspace too small for
// the planned split (or a launch too large to split) runs unsplit, which
// every task must then allow.
int run_grouped(Fmt fmt, int chosen, const GemvArgs* a, int count, int M, void* workspace, size_t workspace_bytes, void* stream) {
    const bool split = workspace != nullptr && workspace_bytes > 0;
    if ((chosen == Q4_VARIANT_TILED || chosen == Q4_VARIANT_SKINNY) && split) {
        const size_t need = grouped_ws_bytes(fmt, chosen, a, count);
        if (need == 0 || workspace_bytes < need) {
            for (int i = 0; i < count; ++i)
                if (chosen == Q4_VARIANT_TILED ? !q4::mm_supported(fmt, M, a[i].K, false) : !q4::skinny_supported(fmt, M, a[i].K, false))
                    return Q4_EVARIANT;
        }
    }
    return run(fmt, chosen, a, count, stream, workspace, workspace_bytes);
}

// Validation of a mixed-format group: fills a[] and fmts[], checks every
// output against every input and the other outputs.
int check_mixed(const q4gemv_mixed_task* tasks, int count, int M, GemvArgs* a, Fmt* fmts, bool* one_launch) {
    if (!tasks) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxTasks) return Q4_EINVAL_SHAPE;
    Range in[q4::kMaxTasks][4], out[q4::kMaxTasks];
    bool stream = M <= 4;
    for (int i = 0; i < count; ++i) {
        const q4gemv_mixed_task& k = tasks[i];
        int rc;
        switch (k.format) {
            case Q4_FMT_Q4G128:
                rc = check_q4(k.x, M, k.K, static_cast<const uint8_t*>(k.weight), static_cast<const uint16_t*>(k.scale), k.minv, k.N,
                              k.y, a[i], in[i], out[i]);
                break;
            case Q4_FMT_NVFP4G16:
                rc = check_nv(k.x, M, k.K, static_cast<const uint8_t*>(k.weight), static_cast<const uint8_t*>(k.scale), k.global_scale,
                              k.N, k.y, a[i], in[i], out[i]);
                break;
            case Q4_FMT_BF16:
                rc = check_bf(k.x, M, k.K, static_cast<const uint16_t*>(k.weight), k.N, k.y, a[i], in[i], out[i]);
                break;
            default:
                return Q4_EINVAL_SHAPE;
        }
        if (rc) return rc;
        fmts[i] = static_cast<Fmt>(k.format);
        stream = stream && q4::stream_supported(fmts[i], M, k.K);
    }
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            for (int r = 0; r < 4; ++r)
                if (overlaps(out[i], in[j][r])) return Q4_EALIAS;
            if (i != j && overlaps(out[i], out[j])) return Q4_EALIAS;
        }
    *one_launch = stream;
    return Q4_OK;
}

// 5 <= M <= 48 and every task on the skinny kernel (with K splits allowed):
// the group can run as one mixed-format skinny launch.
bool mixed_skinny(const GemvArgs* a, const Fmt* fmts, int count, int M) {
    for (int i = 0; i < count; ++i)
        if (!q4::skinny_supported(fmts[i], M, a[i].K, true)) return false;
    return true;
}

// Every task NVFP4 or BF16 and on the tiled kernel (with K splits allowed):
// the group can run as one mixed-format tiled launch.
bool mixed_tiled(const GemvArgs* a, const Fmt* fmts, int count, int M) {
    if (M <= 4) return false;
    for (int i = 0; i < count; ++i)
        if (fmts[i] == q4::kFmtQ4 || pick(fmts[i], Q4_VARIANT_AUTO, M, a[i].N, a[i].K, true) != Q4_VARIANT_TILED) return false;
    return true;
}

// The tasks of format f, in order, and their variant under the automatic
// choice (the grouped calls' rules).
int mixed_subgroup(const GemvArgs* a, const Fmt* fmts, int count, Fmt f, int M, bool split, GemvArgs* sub, int* n, int* chosen) {
    Range in[q4::kMaxTasks][4], out[q4::kMaxTasks];
    *n = 0;
    for (int i = 0; i < count; ++i)
        if (fmts[i] == f) {
            in[*n][0] = in[*n][1] = in[*n][2] = in[*n][3] = Range{0, 0};
            out[*n] = Range{0, 0};   // aliasing was checked across all tasks already
            sub[(*n)++] = a[i];
        }
    if (*n == 0) return Q4_OK;
    return plan_checked(f, sub, in, out, *n, M, Q4_VARIANT_AUTO, split, chosen);
}

// Validation and kernel choice of a fused int4 call (see q4g128_fused_task):
// fills a[] and *tiled (false: the streaming kernel).
int check_fused(const q4g128_fused_task* tasks, int count, int M, bool split, GemvArgs* a, bool* tiled) {
    if (!tasks) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxTasks) return Q4_EINVAL_SHAPE;
    Range in[q4::kMaxTasks][6], out[q4::kMaxTasks];
    bool stream = true, mm = true;
    for (int i = 0; i < count; ++i) {
        const q4g128_fused_task& k = tasks[i];
        int rc = check_q4(k.x, M, k.K, k.qweight, k.scale, k.minv, k.N, k.y, a[i], in[i], out[i]);
        if (rc) return rc;
        in[i][4] = in[i][5] = Range{0, 0};
        if (k.up) {
            if (!aligned(k.up, 16)) return Q4_EALIGN;
            in[i][4] = range_of(k.up, (size_t)M * k.K * 2);
        }
        if (k.residual) {
            if (!aligned(k.residual, 2)) return Q4_EALIGN;
            // a residual that is exactly this task's y is read before each element is written
            if (k.residual != k.y) in[i][5] = range_of(k.residual, (size_t)M * k.N * 2);
        }
        a[i].up = k.up;
        a[i].resid = k.residual;
        stream = stream && M <= 4 && q4::stream_supported(q4::kFmtQ4, M, k.K);
        mm = mm && q4::mm_supported(q4::kFmtQ4, M, k.K, split);
    }
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            for (int r = 0; r < 6; ++r)
                if (overlaps(out[i], in[j][r])) return Q4_EALIAS;
            if (i != j && overlaps(out[i], out[j])) return Q4_EALIAS;
        }
    if (!stream && !mm) return Q4_EVARIANT;
    *tiled = !stream;
    return Q4_OK;
}

// Sampler arguments; `extra` are further input ranges the outputs must avoid.
int check_sample(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u, const int32_t* token,
                 const int32_t* topk_index, const float* topk_prob, const Range* extra, int n_extra) {
    if (!logits || !u || !token) return Q4_EINVAL_PTR;
    if (M < 1 || M > 65535 || V < 1 || V > q4::kMaxVocab || top_k < 1 || top_k > q4::kMaxTopK || top_k > V)
        return Q4_EINVAL_SHAPE;
    if (!(temperature > 0.f) || !(temperature < __builtin_huge_valf())) return Q4_EINVAL_SHAPE;
    if (!aligned(logits, 2) || !aligned(u, 4) || !aligned(token, 4) || (topk_index && !aligned(topk_index, 4)) ||
        (topk_prob && !aligned(topk_prob, 4)))
        return Q4_EALIGN;
    const Range outs[3] = {range_of(token, (size_t)M * 4), topk_index ? range_of(topk_index, (size_t)M * top_k * 4) : Range{0, 0},
                           topk_prob ? range_of(topk_prob, (size_t)M * top_k * 4) : Range{0, 0}};
    const Range ins[2] = {range_of(logits, (size_t)M * V * 2), range_of(u, (size_t)M * 4)};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlaps(outs[i], ins[j])) return Q4_EALIAS;
        for (int j = 0; j < n_extra; ++j)
            if (overlaps(outs[i], extra[j])) return Q4_EALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], outs[j])) return Q4_EALIAS;
    }
    return Q4_OK;
}

}  // namespace

namespace q4 {
LaunchEvents& pending_launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}
}  // namespace q4

extern "C" {

int q4gemv_time_next_launch(void* start_event, void* stop_event) {
    q4::LaunchEvents& ev = q4::pending_launch_events();
    ev.start = reinterpret_cast<hipEvent_t>(start_event);
    ev.stop = reinterpret_cast<hipEvent_t>(stop_event);
    return Q4_OK;
}

int q4g128_gemv_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv,
                        int N, uint16_t* y, int variant, void* stream) {
    GemvArgs a;
    Range in[4], out;
    int rc = check_q4(x, M, K, qweight, scale, minv, N, y, a, in, out);
    if (rc) return rc;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    for (const Range& r : in)
        if (overlaps(out, r)) return Q4_EALIAS;
    const int chosen = pick(q4::kFmtQ4, variant, M, N, K);
    if (chosen < 0) return Q4_EVARIANT;
    return run(q4::kFmtQ4, chosen, a, stream);
}

// Validates an int4 group and picks one kernel family for it.
static int plan_group(const q4g128_task* tasks, int count, int M, int variant, bool split, GemvArgs* a, int* chosen_out) {
    if (!tasks) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxTasks) return Q4_EINVAL_SHAPE;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    Range in[q4::kMaxTasks][4], out[q4::kMaxTasks];
    for (int i = 0; i < count; ++i) {
        const q4g128_task& t = tasks[i];
        int rc = check_q4(t.x, M, t.K, t.qweight, t.scale, t.minv, t.N, t.y, a[i], in[i], out[i]);
        if (rc) return rc;
    }
    return plan_checked(q4::kFmtQ4, a, in, out, count, M, variant, split, chosen_out);
}

int q4g128_gemv_grouped_ws(const q4g128_task* tasks, int count, int M, int variant, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (workspace && !aligned(workspace, 256)) return Q4_EALIGN;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    const bool split = workspace != nullptr && workspace_bytes > 0;
    int rc = plan_group(tasks, count, M, variant, split, a, &chosen);
    if (rc) return rc;
    return run_grouped(q4::kFmtQ4, chosen, a, count, M, workspace, workspace_bytes, stream);
}

int q4g128_gemv_grouped_noalloc(const q4g128_task* tasks, int count, int M, int variant, void* stream) {
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_group(tasks, count, M, variant, true, a, &chosen);
    if (rc) return rc;
    const size_t need = grouped_ws_bytes(q4::kFmtQ4, chosen, a, count);
    if (need > q4::kNoAllocScratchBytes) return Q4_ESCRATCH;
    void* ws = nullptr;
    if (need > 0 && q4::noalloc_scratch(reinterpret_cast<hipStream_t>(stream), &ws) != hipSuccess) return Q4_ELAUNCH;
    return run_grouped(q4::kFmtQ4, chosen, a, count, M, ws, ws ? q4::kNoAllocScratchBytes : 0, stream);
}

int q4g128_gemv_grouped(const q4g128_task* tasks, int count, int M, int variant, void* stream) {
    return q4g128_gemv_grouped_ws(tasks, count, M, variant, nullptr, 0, stream);
}

int q4g128_workspace_bytes(const q4g128_task* tasks, int count, int M, size_t* bytes) {
    if (!bytes) return Q4_EINVAL_PTR;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_group(tasks, count, M, Q4_VARIANT_AUTO, true, a, &chosen);
    if (rc) return rc;
    *bytes = grouped_ws_bytes(q4::kFmtQ4, chosen, a, count);
    return Q4_OK;
}

int q4g128_gemv(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N,
                uint16_t* y, void* stream) {
    return q4g128_gemv_variant(x, M, K, qweight, scale, minv, N, y, Q4_VARIANT_AUTO, stream);
}

int nvfp4g16_gemv_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale,
                          int N, uint16_t* y, int variant, void* stream) {
    int rc = check_common(x, M, K, N, y);
    if (rc) return rc;
    if (!qweight || !scale_e4m3) return Q4_EINVAL_PTR;
    if (K % 32) return Q4_EINVAL_SHAPE;
    if (!aligned(qweight, 16)) return Q4_EALIGN;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    const Range yr = range_of(y, (size_t)M * N * 2);
    if (overlaps(yr, range_of(x, (size_t)M * K * 2)) || overlaps(yr, range_of(qweight, (size_t)N * K / 2)) ||
        overlaps(yr, range_of(scale_e4m3, (size_t)N * K / 16)))
        return Q4_EALIAS;
    const int chosen = pick(q4::kFmtNvfp4, variant, M, N, K);
    if (chosen < 0) return Q4_EVARIANT;
    GemvArgs a{};
    a.x = x; a.w = qweight; a.scale8 = scale_e4m3; a.gscale = global_scale; a.y = y; a.M = M; a.N = N; a.K = K;
    return run(q4::kFmtNvfp4, chosen, a, stream);
}

int nvfp4g16_gemv(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale, int N,
                  uint16_t* y, void* stream) {
    return nvfp4g16_gemv_variant(x, M, K, qweight, scale_e4m3, global_scale, N, y, Q4_VARIANT_AUTO, stream);
}

int bf16_gemv_variant(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* y, int variant, void* stream) {
    int rc = check_common(x, M, K, N, y);
    if (rc) return rc;
    if (!w) return Q4_EINVAL_PTR;
    if (K % 8) return Q4_EINVAL_SHAPE;
    if (!aligned(w, 16)) return Q4_EALIGN;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    const Range yr = range_of(y, (size_t)M * N * 2);
    if (overlaps(yr, range_of(x, (size_t)M * K * 2)) || overlaps(yr, range_of(w, (size_t)N * K * 2))) return Q4_EALIAS;
    const int chosen = pick(q4::kFmtBf16, variant, M, N, K);
    if (chosen < 0) return Q4_EVARIANT;
    GemvArgs a{};
    a.x = x; a.w = reinterpret_cast<const uint8_t*>(w); a.y = y; a.M = M; a.N = N; a.K = K;
    return run(q4::kFmtBf16, chosen, a, stream);
}

int bf16_gemv(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* y, void* stream) {
    return bf16_gemv_variant(x, M, K, w, N, y, Q4_VARIANT_AUTO, stream);
}

static int plan_nv(const nvfp4g16_task* tasks, int count, int M, int variant, bool split, GemvArgs* a, int* chosen) {
    if (!tasks) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxTasks) return Q4_EINVAL_SHAPE;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    Range in[q4::kMaxTasks][4], out[q4::kMaxTasks];
    for (int i = 0; i < count; ++i) {
        const nvfp4g16_task& t = tasks[i];
        int rc = check_nv(t.x, M, t.K, t.qweight, t.scale_e4m3, t.global_scale, t.N, t.y, a[i], in[i], out[i]);
        if (rc) return rc;
    }
    return plan_checked(q4::kFmtNvfp4, a, in, out, count, M, variant, split, chosen);
}

int nvfp4g16_gemv_grouped_ws(const nvfp4g16_task* tasks, int count, int M, int variant, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (workspace && !aligned(workspace, 256)) return Q4_EALIGN;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_nv(tasks, count, M, variant, workspace != nullptr && workspace_bytes > 0, a, &chosen);
    if (rc) return rc;
    return run_grouped(q4::kFmtNvfp4, chosen, a, count, M, workspace, workspace_bytes, stream);
}

int nvfp4g16_workspace_bytes(const nvfp4g16_task* tasks, int count, int M, size_t* bytes) {
    if (!bytes) return Q4_EINVAL_PTR;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_nv(tasks, count, M, Q4_VARIANT_AUTO, true, a, &chosen);
    if (rc) return rc;
    *bytes = grouped_ws_bytes(q4::kFmtNvfp4, chosen, a, count);
    return Q4_OK;
}

static int plan_bf(const bf16_task* tasks, int count, int M, int variant, bool split, GemvArgs* a, int* chosen) {
    if (!tasks) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxTasks) return Q4_EINVAL_SHAPE;
    if (!variant_ok(variant)) return Q4_EVARIANT;
    Range in[q4::kMaxTasks][4], out[q4::kMaxTasks];
    for (int i = 0; i < count; ++i) {
        const bf16_task& t = tasks[i];
        int rc = check_bf(t.x, M, t.K, t.w, t.N, t.y, a[i], in[i], out[i]);
        if (rc) return rc;
    }
    return plan_checked(q4::kFmtBf16, a, in, out, count, M, variant, split, chosen);
}

int bf16_gemv_grouped_ws(const bf16_task* tasks, int count, int M, int variant, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (workspace && !aligned(workspace, 256)) return Q4_EALIGN;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_bf(tasks, count, M, variant, workspace != nullptr && workspace_bytes > 0, a, &chosen);
    if (rc) return rc;
    return run_grouped(q4::kFmtBf16, chosen, a, count, M, workspace, workspace_bytes, stream);
}

int bf16_workspace_bytes(const bf16_task* tasks, int count, int M, size_t* bytes) {
    if (!bytes) return Q4_EINVAL_PTR;
    GemvArgs a[q4::kMaxTasks];
    int chosen = 0;
    int rc = plan_bf(tasks, count, M, Q4_VARIANT_AUTO, true, a, &chosen);
    if (rc) return rc;
    *bytes = grouped_ws_bytes(q4::kFmtBf16, chosen, a, count);
    return Q4_OK;
}

int q4g128_dequant_f32(const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N, int K, float* w, void* stream) {
    if (!qweight || !scale || !minv || !w) return Q4_EINVAL_PTR;
    if (N < 1 || N > kMaxN || K < 128 || K > kMaxK || K % 128) return Q4_EINVAL_SHAPE;
    if (!aligned(qweight, 16) || !aligned(scale, 2) || !aligned(minv, 2) || !aligned(w, 16)) return Q4_EALIGN;
    const size_t G = (size_t)K / 128;
    const Range wr = range_of(w, (size_t)N * K * 4);
    if (overlaps(wr, range_of(qweight, (size_t)N * K / 2)) || overlaps(wr, range_of(scale, (size_t)N * G * 2)) ||
        overlaps(wr, range_of(minv, (size_t)N * G * 2)))
        return Q4_EALIAS;
    hipError_t e = q4::launch_q4_dequant(qweight, scale, minv, N, K, w, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

int nvfp4g16_dequant_f32(const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale, int N, int K, float* w,
                         void* stream) {
    if (!qweight || !scale_e4m3 || !w) return Q4_EINVAL_PTR;
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || K % 32) return Q4_EINVAL_SHAPE;
    if (!aligned(qweight, 16) || !aligned(w, 16)) return Q4_EALIGN;
    const Range wr = range_of(w, (size_t)N * K * 4);
    if (overlaps(wr, range_of(qweight, (size_t)N * K / 2)) || overlaps(wr, range_of(scale_e4m3, (size_t)N * K / 16)))
        return Q4_EALIAS;
    hipError_t e = q4::launch_nvfp4_dequant(qweight, scale_e4m3, global_scale, N, K, w, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

// Workspace of a fused tiled call: the split-K part, then (256-byte aligned)
// one h buffer per gated task.
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
// h starts after the split-K part, and in any case past the arrival counters
// The fused tiled-path plan: split-K workspace of the tiled kernel and, where
// every task qualifies for the skinny kernel at this M (a workspace given),
// of the skinny kernel; true if the skinny kernel may run.
bool fused_skinny_ok(const GemvArgs* a, int count, int M, bool split, size_t* need_mm, size_t* need_sk) {
    *need_mm = q4::mm_workspace_bytes(q4::kFmtQ4, a, count);
    *need_sk = 0;
    bool ok = split && M >= 5 && M <= q4::kSkinnyMaxM;
    for (int i = 0; i < count && ok; ++i) ok = q4::skinny_supported(M, a[i].K, true);
    if (ok) *need_sk = q4::skinny_workspace_bytes(a, count);
    return ok;
}

size_t fused_h_offset(size_t need) { return align256(need > q4::kWsCounterBytes ? need : q4::kWsCounterBytes); }
size_t fused_h_bytes(const GemvArgs* a, int count) {
    size_t n = 0;
    for (int i = 0; i < count; ++i)
        if (a[i].up) n += align256((size_t)a[i].M * a[i].K * 2);
    return n;
}

int q4gemv_grouped_mixed(const q4gemv_mixed_task* tasks, int count, int M, void* workspace, size_t workspace_bytes,
                         void* stream) {
    GemvArgs a[q4::kMaxTasks];
    Fmt fmts[q4::kMaxTasks];
    bool one = false;
    int rc = check_mixed(tasks, count, M, a, fmts, &one);
    if (rc) return rc;
    if (one) {
        hipError_t e = q4::launch_stream_mixed(fmts, a, count, reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
    }
    const bool split = workspace != nullptr && workspace_bytes > 0;
    if (mixed_skinny(a, fmts, count, M)) {
        const size_t need = q4::skinny_workspace_bytes(fmts, a, count);
        bool unsplit_ok = true;
        for (int i = 0; i < count; ++i) unsplit_ok = unsplit_ok && q4::skinny_supported(fmts[i], M, a[i].K, false);
        if ((split && need <= workspace_bytes) || unsplit_ok) {
            hipError_t e = q4::launch_skinny(fmts, a, count, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
            return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
        }
    }
    if (split && mixed_tiled(a, fmts, count, M)) {
        const size_t need = q4::mm_workspace_bytes(q4::kFmtNvfp4, a, count);
        if (need <= workspace_bytes) {
            hipError_t e = q4::launch_mm_mixed(fmts, a, count, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
            return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
        }
    }
    // one grouped launch per format, in order of first appearance; every
    // subgroup is planned before anything is enqueued
    Fmt order[3];
    int nf = 0;
    for (int i = 0; i < count; ++i) {
        bool seen = false;
        for (int j = 0; j < nf; ++j) seen = seen || order[j] == fmts[i];
        if (!seen) order[nf++] = fmts[i];
    }
    GemvArgs sub[3][q4::kMaxTasks];
    int n[3], chosen[3];
    for (int f = 0; f < nf; ++f) {
        rc = mixed_subgroup(a, fmts, count, order[f], M, split, sub[f], &n[f], &chosen[f]);
        if (rc) return rc;
        if ((chosen[f] == Q4_VARIANT_TILED || chosen[f] == Q4_VARIANT_SKINNY) && split) {
            const size_t need = grouped_ws_bytes(order[f], chosen[f], sub[f], n[f]);
            if (need == 0 || workspace_bytes < need)
                for (int i = 0; i < n[f]; ++i)
                    if (chosen[f] == Q4_VARIANT_TILED ? !q4::mm_supported(order[f], M, sub[f][i].K, false)
                                                      : !q4::skinny_supported(order[f], M, sub[f][i].K, false))
                        return Q4_EVARIANT;
        }
    }
    for (int f = 0; f < nf; ++f) {
        rc = run_grouped(order[f], chosen[f], sub[f], n[f], M, workspace, workspace_bytes, stream);
        if (rc) return rc;
    }
    return Q4_OK;
}

int q4gemv_mixed_workspace_bytes(const q4gemv_mixed_task* tasks, int count, int M, size_t* bytes) {
    if (!bytes) return Q4_EINVAL_PTR;
    GemvArgs a[q4::kMaxTasks];
    Fmt fmts[q4::kMaxTasks];
    bool one = false;
    int rc = check_mixed(tasks, count, M, a, fmts, &one);
    if (rc) return rc;
    size_t need = 0;
    if (!one && mixed_skinny(a, fmts, count, M)) need = q4::skinny_workspace_bytes(fmts, a, count);
    if (!one && mixed_tiled(a, fmts, count, M)) {
        const size_t b = q4::mm_workspace_bytes(q4::kFmtNvfp4, a, count);
        need = b > need ? b : need;
    }
    if (!one) {
        for (int f = 0; f < 3; ++f) {
            GemvArgs sub[q4::kMaxTasks];
            int n = 0, chosen = 0;
            rc = mixed_subgroup(a, fmts, count, static_cast<Fmt>(f), M, true, sub, &n, &chosen);
            if (rc) return rc;
            if (n) {
                const size_t b = grouped_ws_bytes(static_cast<Fmt>(f), chosen, sub, n);
                need = b > need ? b : need;
            }
        }
    }
    *bytes = need;
    return Q4_OK;
}

int q4g128_gemv_fused(const q4g128_fused_task* tasks, int count, int M, void* workspace, size_t workspace_bytes, void* stream) {
    GemvArgs a[q4::kMaxTasks];
    bool tiled = false;
    const bool split = workspace != nullptr && workspace_bytes > 0;
    if (workspace && !aligned(workspace, 256)) return Q4_EALIGN;
    int rc = check_fused(tasks, count, M, split, a, &tiled);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (!tiled) {
        e = q4::launch_stream_fused(a, count, s);
        return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
    }
    // Everything is planned and checked before the first enqueue.  The h
    // buffers start past the split-K part and never below the counter region,
    // which other calls on the same workspace rely on staying zero.  With a
    // workspace, 5 <= M <= 48 runs on the skinny kernel (residual epilogue;
    // gated tasks read the h formed in the pass); otherwise the tiled kernel,
    // which can also form h in its loader.
    size_t need_mm = 0, need_sk = 0;
    const bool sk_ok = fused_skinny_ok(a, count, M, split, &need_mm, &need_sk);
    const size_t need = need_mm > need_sk ? need_mm : need_sk;
    const size_t h_off = fused_h_offset(need), h_bytes = fused_h_bytes(a, count);
    const bool form_h = split && h_bytes > 0 && workspace_bytes >= h_off + h_bytes;
    const size_t mm_bytes = form_h ? h_off : workspace_bytes;
    const bool use_sk = sk_ok && (h_bytes == 0 || form_h) && (need_sk == 0 || mm_bytes >= need_sk);
    if (!use_sk && split && (need_mm == 0 || mm_bytes < need_mm)) {
        for (int i = 0; i < count; ++i)
            if (!q4::mm_supported(q4::kFmtQ4, M, a[i].K, false)) return Q4_EVARIANT;
    }
    if (form_h) {
        // h formed once into the workspace; the tiled kernel reads it as x
        const uint16_t* g[q4::kMaxTasks];
        const uint16_t* u[q4::kMaxTasks];
        uint16_t* h[q4::kMaxTasks];
        size_t n[q4::kMaxTasks];
        int ng = 0;
        uint8_t* p = static_cast<uint8_t*>(workspace) + h_off;
        for (int i = 0; i < count; ++i) {
            if (!a[i].up) continue;
            g[ng] = a[i].x; u[ng] = a[i].up; h[ng] = reinterpret_cast<uint16_t*>(p);
            n[ng] = (size_t)M * a[i].K;
            a[i].x = h[ng];
            a[i].up = nullptr;
            p += align256(n[ng] * 2);
            ++ng;
        }
        if (q4::launch_silu_mul(g, u, h, n, ng, s) != hipSuccess) return Q4_ELAUNCH;
    }
    e = use_sk ? q4::launch_skinny(a, count, workspace, mm_bytes, s) : q4::launch_mm_fused(a, count, workspace, mm_bytes, s);
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

int q4g128_fused_workspace_bytes(const q4g128_fused_task* tasks, int count, int M, size_t* bytes) {
    if (!bytes) return Q4_EINVAL_PTR;
    GemvArgs a[q4::kMaxTasks];
    bool tiled = false;
    int rc = check_fused(tasks, count, M, true, a, &tiled);
    if (rc) return rc;
    if (!tiled) {
        *bytes = 0;
        return Q4_OK;
    }
    size_t need_mm = 0, need_sk = 0;
    fused_skinny_ok(a, count, M, true, &need_mm, &need_sk);
    const size_t need = need_mm > need_sk ? need_mm : need_sk;
    const size_t h_bytes = fused_h_bytes(a, count);
    *bytes = h_bytes ? fused_h_offset(need) + h_bytes : need;
    return Q4_OK;
}

int q4g128_gemm_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv,
                        int N, uint16_t* y, int variant, void* stream) {
    if (variant != Q4_VARIANT_AUTO && variant != Q4_VARIANT_TILED && variant != Q4_VARIANT_GEMM) return Q4_EVARIANT;
    if (variant == Q4_VARIANT_AUTO && M >= 1 && M <= kMaxM)
        return q4g128_gemv_variant(x, M, K, qweight, scale, minv, N, y, Q4_VARIANT_AUTO, stream);
    if (M < 1 || M > (1 << 19)) return Q4_EINVAL_SHAPE;
    GemvArgs a;
    Range in[4], out;
    int rc = check_q4(x, 1, K, qweight, scale, minv, N, y, a, in, out);   // pointers, K, N, alignment
    if (rc) return rc;
    in[0] = range_of(x, (size_t)M * K * 2);
    out = range_of(y, (size_t)M * N * 2);
    for (int r = 0; r < 4; ++r)
        if (overlaps(out, in[r])) return Q4_EALIAS;
    a.M = M;
    int chosen = variant;
    if (chosen == Q4_VARIANT_AUTO)
        chosen = (q4::gemm_tiles(M, N, 2) >= kGemmMinTiles || !q4::mm_chunks_supported(K)) ? Q4_VARIANT_GEMM : Q4_VARIANT_TILED;
    hipError_t e;
    if (chosen == Q4_VARIANT_TILED) {
        if (!q4::mm_chunks_supported(K)) return Q4_EVARIANT;
        e = q4::launch_mm_chunks(a, reinterpret_cast<hipStream_t>(stream));
    } else {
        if (K >= (1 << 24)) return Q4_EVARIANT;
        e = q4::launch_gemm(a, q4::gemm_tile_nt(M, N), reinterpret_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

int q4g128_gemm(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N,
                uint16_t* y, void* stream) {
    return q4g128_gemm_variant(x, M, K, qweight, scale, minv, N, y, Q4_VARIANT_AUTO, stream);
}

int q4_sample_topk(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u, int32_t* token,
                   int32_t* topk_index, float* topk_prob, void* stream) {
    int rc = check_sample(logits, M, V, temperature, top_k, u, token, topk_index, topk_prob, nullptr, 0);
    if (rc) return rc;
    hipError_t e = q4::launch_topk_sample(logits, M, V, temperature, top_k, u, token, topk_index, topk_prob,
                                          reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

int bf16_head_sample(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* logits, float temperature, int top_k,
                     const float* u, int32_t* token, int32_t* topk_index, float* topk_prob, void* stream) {
    GemvArgs a;
    Range in[4], out;
    int rc = check_bf(x, M, K, w, N, logits, a, in, out);
    if (rc) return rc;
    for (int r = 0; r < 2; ++r)
        if (overlaps(out, in[r])) return Q4_EALIAS;
    // the GEMV writes the logits before the sampler reads u
    if (u && overlaps(out, range_of(u, (size_t)M * 4))) return Q4_EALIAS;
    rc = check_sample(logits, M, N, temperature, top_k, u, token, topk_index, topk_prob, in, 2);
    if (rc) return rc;
    const int chosen = pick(q4::kFmtBf16, Q4_VARIANT_AUTO, M, N, K);
    if (chosen < 0) return Q4_EVARIANT;
    rc = run(q4::kFmtBf16, chosen, a, stream);
    if (rc) return rc;
    hipError_t e = q4::launch_topk_sample(logits, M, N, temperature, top_k, u, token, topk_index, topk_prob,
                                          reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

size_t bf16_head_sample_workspace_bytes(int M, int N, int K, int top_k) {
    if (M < 1 || M > kMaxM || N < 1 || K < 1 || top_k < 1 || top_k > N || top_k > q4::kMaxTopK || N > q4::kMaxVocab) return 0;
    // one row: GEMV and sampling in one launch; a batch: the GEMV, then the
    // sampler split over blocks of each row (a row of one block gains nothing)
    if (M == 1) return q4::head_sample_workspace_bytes(M, N, K, top_k);
    return N > q4::kSplitBlock ? q4::topk_sample_split_ws_bytes(M, N, top_k) : 0;
}

int bf16_head_sample_ws(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* logits, float temperature, int top_k,
                        const float* u, int32_t* token, int32_t* topk_index, float* topk_prob, void* workspace, size_t ws_bytes,
                        void* stream) {
    const size_t need = bf16_head_sample_workspace_bytes(M, N, K, top_k);
    if (need == 0 || workspace == nullptr || ws_bytes < need)
        return bf16_head_sample(x, M, K, w, N, logits, temperature, top_k, u, token, topk_index, topk_prob, stream);
    GemvArgs a;
    Range in[4], out;
    int rc = check_bf(x, M, K, w, N, logits, a, in, out);
    if (rc) return rc;
    for (int r = 0; r < 2; ++r)
        if (overlaps(out, in[r])) return Q4_EALIAS;
    if (u && overlaps(out, range_of(u, (size_t)M * 4))) return Q4_EALIAS;
    rc = check_sample(logits, M, N, temperature, top_k, u, token, topk_index, topk_prob, in, 2);
    if (rc) return rc;
    if (!aligned(workspace, 4)) return Q4_EALIGN;
    const Range wr = range_of(workspace, need);
    const Range others[7] = {in[0], in[1], out, range_of(u, (size_t)M * 4), range_of(token, (size_t)M * 4),
                             topk_index ? range_of(topk_index, (size_t)M * top_k * 4) : Range{0, 0},
                             topk_prob ? range_of(topk_prob, (size_t)M * top_k * 4) : Range{0, 0}};
    for (const Range& r : others)
        if (overlaps(wr, r)) return Q4_EALIAS;
    if (M == 1) {
        hipError_t e = q4::launch_head_sample(a, temperature, top_k, u, token, topk_index, topk_prob, workspace,
                                              reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
    }
    const int chosen = pick(q4::kFmtBf16, Q4_VARIANT_AUTO, M, N, K);
    if (chosen < 0) return Q4_EVARIANT;
    rc = run(q4::kFmtBf16, chosen, a, stream);
    if (rc) return rc;
    hipError_t e = q4::launch_topk_sample_split(logits, M, N, temperature, top_k, u, token, topk_index, topk_prob, workspace,
                                                reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

size_t q4gemv_stream_read_sink_words(const size_t* bytes, int count) {
    if (!bytes || count < 1 || count > q4::kMaxReadBufs) return 0;
    for (int i = 0; i < count; ++i)
        if (bytes[i] < 16 || bytes[i] >= ((size_t)1 << 32)) return 0;
    return q4::stream_read_sink_words(bytes, count);
}

int q4gemv_stream_read(const void* const* bufs, const size_t* bytes, int count, uint32_t* sink, size_t sink_words,
                       void* stream) {
    if (!bufs || !bytes || !sink) return Q4_EINVAL_PTR;
    if (count < 1 || count > q4::kMaxReadBufs) return Q4_EINVAL_SHAPE;
    for (int i = 0; i < count; ++i) {
        if (!bufs[i]) return Q4_EINVAL_PTR;
        if (bytes[i] < 16 || bytes[i] >= ((size_t)1 << 32)) return Q4_EINVAL_SHAPE;
        if (!aligned(bufs[i], 4)) return Q4_EALIGN;
    }
    const size_t need = q4::stream_read_sink_words(bytes, count);
    if (sink_words < need) return Q4_EINVAL_SHAPE;
    if (!aligned(sink, 4)) return Q4_EALIGN;
    const Range sr = range_of(sink, need * 4);
    for (int i = 0; i < count; ++i)
        if (overlaps(sr, range_of(bufs[i], bytes[i]))) return Q4_EALIAS;
    hipError_t e = q4::launch_stream_read(bufs, bytes, count, sink, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q4_OK : Q4_ELAUNCH;
}

const char* q4gemv_variant_name(int fmt, int variant, int M, int N, int K) {
    if (fmt < Q4_FMT_Q4G128 || fmt > Q4_FMT_BF16 || !variant_ok(variant) || M < 1 || M > kMaxM || K < 1) return "invalid";
    const int c = pick(static_cast<Fmt>(fmt), variant, M, N, K);
    if (c == Q4_VARIANT_DOT2) return "dot2";
    if (c == Q4_VARIANT_MFMA) return "mfma";
    if (c == Q4_VARIANT_STREAM) return "stream";
    if (c == Q4_VARIANT_TILED) return "tiled";
    if (c == Q4_VARIANT_SKINNY) return "skinny";
    return "invalid";
}

const char* q4gemv_strerror(int status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_EINVAL_PTR: return "null pointer argument";
        case Q4_EINVAL_SHAPE: return "M, N or K out of range for this format";
        case Q4_EALIGN: return "misaligned pointer";
        case Q4_EALIAS: return "output overlaps an input";
        case Q4_ELAUNCH: return "kernel launch failed";
        case Q4_EVARIANT: return "unknown variant or variant cannot run this shape";
        case Q4_ESCRATCH: return "the call needs more split-K scratch than the built-in array holds";
        default: return "unknown status";
    }
}

int q4gemv_version(void) { return 110; }

}  // extern "C"
