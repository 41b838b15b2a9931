// C ABI of the FP4 GEMM (include/fp4gemm.h): argument checks, shape choice and
// launches.  The kernels are in kernels.h; the decode and prefill kernels are
// instantiated in their own translation units (dispatch.h).
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "dispatch.h"
#include "kernels.h"

int fp4_check_weight_shape(int64_t N, int64_t K, int format);  // repack.cpp

namespace fp4 {

std::atomic<int> g_device_state[64];  // 0 unknown, 1 gfx950, 2 other

static int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP4_ERR_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FP4_ERR_DEVICE;
        st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? FP4_OK : FP4_ERR_DEVICE;
}

static int launch_status() {
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// Row block the kernels for this m read A in (A offsets are 32-bit).
static int64_t a_row_block(int64_t M) {
    if (M <= 16) return 16;
    if (M <= 32) return 32;
    if (M <= 64) return 64;
    return 128;  // prefill m-block
}

// Tuning override, read once per process.
static DecodeShape decode_override() {
    static const DecodeShape ov = [] {
        DecodeShape d{0, 0, 0, 0};
        const char* e = getenv("FP4GEMM_DECODE");
        if (e && *e) sscanf(e, "%d,%d,%d,%d", &d.tn, &d.nwn, &d.nwk, &d.s);
        return d;
    }();
    return ov;
}

static bool decode_compiled(int MB, const DecodeShape& d);

struct DecodeCand {
    int mb, tn, nwn, nwk;
};
static const DecodeCand* decode_shapes(int* count);

constexpr int kCUs = 256;  // compute units of an MI355X / MI350X (gfx950)

// Modelled time of one decode launch (seconds), from measurements on MI355X:
// a compute unit streams about 22 GB/s of weights when all 256 are busy;
// activations are L2 hits and cost about half a weight byte per real row
// (rows past m read nothing); every workgroup pays ~1.5 us before its first
// block arrives; a CU needs ~24 KiB of code blocks in flight (three chunks
// ahead per wave) to cover the memory latency; a K split over S workgroups
// adds the partial sums' round trip, the arrival count and the last
// workgroup's pass over the partials (~5 us in all, fit to the measured
// shapes).
static double decode_cost(int fmt, int MB, int64_t M, int64_t N, int NT, int SB, const DecodeShape& d) {
    const int g = d.tn * d.nwn;
    const int groups = (NT + g - 1) / g;
    const int wgs = groups * d.s;
    const int per_cu = (wgs + kCUs - 1) / kCUs;
    const int bpw = (SB + d.s - 1) / d.s;
    const int waves = d.nwn * d.nwk;
    const int resident = std::max(1, std::min(per_cu, 16 / waves));
    const double rows = (double)std::min<int64_t>(M, 16 * MB);
    const double tile_block = fmt == 0 ? 4608.0 : 4352.0;  // code + scale bytes per tile per 512-K block
    const double bytes = per_cu * ((double)g * bpw * tile_block + rows * bpw * 1024.0 * 0.5);
    double t = bytes / 22e9 + ((per_cu + resident - 1) / resident) * 1.5e-6;
    const double inflight = (double)waves * resident * d.tn * 3.0 * 1024.0;
    if (inflight < 24.0 * 1024.0) t *= 24.0 * 1024.0 / inflight;
    if (d.s > 1) t += 5e-6 + 2.0 * d.s * (double)M * (double)N * 4.0 / 2e12;
    // Ties between shapes that move the same bytes: fewer tiles per wave
    // (shorter dependency chains) and more K groups (the waves of a group
    // share one activation stream) measure slightly faster.
    return t * (1.0 + 0.03 * (d.tn - 1)) * (1.0 - 0.01 * (d.nwk - 1));
}

// Shape for m <= 16 * MB: the compiled shape and K split with the least
// modelled time (FP4GEMM_DECODE="TN,NWN,NWK,S" overrides it for tuning).
static DecodeShape pick_decode(int fmt, int MB, int64_t M, int64_t N, int NT, int SB) {
    DecodeShape d = decode_override();
    if (d.tn > 0 && decode_compiled(MB, d)) {
        d.s = d.s < 1 ? 1 : (d.s > SB ? SB : d.s);
        if (M * N >= (int64_t(1) << 29)) d.s = 1;
        return d;
    }
    int count = 0;
    const DecodeCand* c = decode_shapes(&count);
    DecodeShape best{0, 0, 0, 1};
    double best_t = 1e30;
    for (int i = 0; i < count; ++i) {
        if (c[i].mb != MB) continue;
        for (int S : {1, 2, 4, 8, 16}) {
            if (S > SB || (S > 1 && M * N >= (int64_t(1) << 29))) break;  // partial planes use 32-bit offsets
            const DecodeShape cand{c[i].tn, c[i].nwn, c[i].nwk, S};
            if (c[i].nwk > (SB + S - 1) / S) continue;  // every K group gets a block
            const double t = decode_cost(fmt, MB, M, N, NT, SB, cand);
            if (t < best_t) {
                best_t = t;
                best = cand;
            }
        }
    }
    return best;
}

// K split: S partial planes of M x N FP32, then one 8-byte arrival word per
// workgroup group (split_counter_floats in kernels.h).
static size_t decode_workspace_bytes(const DecodeShape& d, int64_t M, int64_t N, int NT) {
    if (d.s <= 1) return 0;
    const int groups = (NT + d.tn * d.nwn - 1) / (d.tn * d.nwn);
    return split_counter_floats(d.s, int(M), int(N)) * sizeof(float) + (size_t)groups * 8;
}

// Launch tags of the split-K arrival words: unique per launch (never 0).
static std::atomic<uint32_t> g_split_tag{0};
static uint32_t next_split_tag() {
    uint32_t t;
    do t = g_split_tag.fetch_add(1, std::memory_order_relaxed) + 1;
    while (t == 0);
    return t;
}

static const DecodeCand* decode_shapes(int* count) {
#define FP4_DECODE_ENTRY(MB_, TN_, NWN_, NWK_) {MB_, TN_, NWN_, NWK_},
    static const DecodeCand table[] = {FP4_DECODE_SHAPES(FP4_DECODE_ENTRY)};
#undef FP4_DECODE_ENTRY
    *count = int(sizeof(table) / sizeof(table[0]));
    return table;
}

static bool decode_compiled(int MB, const DecodeShape& d) {
#define FP4_DECODE_HAS(MB_, TN_, NWN_, NWK_) \
    if (MB == MB_ && d.tn == TN_ && d.nwn == NWN_ && d.nwk == NWK_) return true;
    FP4_DECODE_SHAPES(FP4_DECODE_HAS)
#undef FP4_DECODE_HAS
    return false;
}

static void launch_reduce(int act, const float* P, void* C, int64_t total, int S, float alpha, hipStream_t s) {
    const int64_t threads = (total + 3) / 4;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (act == 0)
        reduce_partials<0><<<grid, block, 0, s>>>(P, (uint16_t*)C, total, S, alpha);
    else
        reduce_partials<1><<<grid, block, 0, s>>>(P, (uint16_t*)C, total, S, alpha);
}

// Tuning override, read once per process.
static PrefillShape prefill_override() {
    static const PrefillShape ov = [] {
        PrefillShape t{0, 0, 0, 0, 1};
        const char* e = getenv("FP4GEMM_PREFILL");
        if (e && *e) sscanf(e, "%d,%d,%d,%d,%d", &t.wm, &t.wn, &t.mbw, &t.tnw, &t.s);
        return t;
    }();
    return ov;
}

static bool prefill_compiled(const PrefillShape& t) {
#define FP4_PREFILL_HAS(WM_, WN_, MBW_, TNW_) \
    if (t.wm == WM_ && t.wn == WN_ && t.mbw == MBW_ && t.tnw == TNW_) return true;
    FP4_PREFILL_SHAPES(FP4_PREFILL_HAS)
#undef FP4_PREFILL_HAS
    return false;
}

// Measured on MI355X over the Llama-3-70B prefill shapes (m = 256): eight
// waves (two per SIMD), each over all 128 rows of the block with two
// n-tiles, so each dequantized fragment feeds 8 products and one wave's
// vector work overlaps the other's matrix work (about 10 % faster than four
// waves of four n-tiles); the K split S minimizes the rounds of workgroups
// per unit of work (QKV 3, O and down 4 at m = 256).  Where m > 128 and the
// 128-row tiles take more than one round without a split, 256-row tiles
// (gemm_prefill_tall: eight waves of 16 m-blocks x 2 n-tiles, each weight
// dequantized once per 256 rows) can cover the layer in fewer rounds: gate_up
// 57344 x 8192 at m = 256 runs 224 tall workgroups in one round against 448
// of 128 rows in two (MI355X, 60 launches back to back, the two plans
// interleaved: 204.5 against 218.9 us; at m = 512 388.8 against 418.7 us;
// same outputs bit for bit).  A tall round does the work of two 128-row
// rounds in about 1.86 times the time; at m = 256 the split layers stay on
// 128-row tiles (QKV 55.1 against 61.4 us for tall tiles with S = 6, O 46.2
// against 57.7, down 111.8 against 116.3 with S = 8).  128 x 128 tiles with a smaller split measured faster on
// down on one box (121 against 128 us) and slower on another (142 against
// 127 us), so they are not picked.  FP4GEMM_PREFILL="WM,WN,MBW,TNW,S"
// overrides the pick.
static PrefillShape pick_prefill(int fmt, int64_t M, int64_t N, int NT, int SB) {
    (void)fmt;
    (void)N;
    PrefillShape t = prefill_override();
    if (t.wm > 0 && prefill_compiled(t)) {
        t.s = t.s < 1 ? 1 : (t.s > SB ? SB : t.s);
        return t;
    }
    // Time model fit to MI355X (m = 256): one workgroup per CU at a time
    // (eight waves); a round of 128 x 256 workgroups over the whole K takes
    // about 17 ns per K element (a round of 256 x 256 ones 1.86 times that),
    // so a K split S runs ceil(blocks * S / 256) rounds of 1/S of that; a
    // split also writes and reads S FP32 partials per output (about 5 TB/s)
    // and pays the reduce launch (about 5 us).
    struct Cand {
        PrefillShape shape;
        int64_t blocks;
        double t_round;
    };
    const double t_round = 0.017e-6 * double(SB) * kScaleBlockK;
    const int NG = (NT + 15) / 16;
    const Cand cands[2] = {{PrefillShape{1, 8, 8, 2, 1}, ((M + 127) / 128) * NG, t_round},
                           {PrefillShape{1, 8, 16, 2, 1}, ((M + 255) / 256) * NG, 1.86 * t_round}};
    const int ncand = M > 128 ? 2 : 1;
    double best = 1e30;
    for (int c = 0; c < ncand; ++c)
        for (int s = 1; s <= 8 && s <= SB; ++s) {
            const double rounds = double((cands[c].blocks * s + kCUs - 1) / kCUs);
            const double split = s > 1 ? 5e-6 + double(s) * double(M) * double(N) * 8.0 / 5e12 : 0.0;
            const double cost = rounds * cands[c].t_round / s + split;
            if (cost < best - 1e-9) {
                best = cost;
                t = cands[c].shape;
                t.s = s;
            }
        }
    return t;
}

// 33 <= m <= 64 on a wide layer (at least 128 groups of 256 columns, enough
// to fill the GPU without a K split): the prefill kernel with 64-row tiles
// (eight waves of 4 m-blocks x 2 n-tiles, whole K) beats the 64-row decode
// kernel, whose activation re-reads equal its weight bytes there (MI355X,
// 57344 x 8192: 88 against 128 us at m = 64, 82 against 110 us at m = 33).
// Narrower layers measured no consistent winner and keep the decode kernel.
static bool wide_mid_m(int64_t M, int NT) {
    return M > 32 && M <= 64 && (NT + 15) / 16 >= 128;
}

// 33 <= m <= 64 on narrower layers: the prefill kernel with 64-row tiles
// (eight waves of 4 m-blocks x 2 n-tiles) and a K split over one round of
// workgroups, instead of the 64-row decode kernel, when the decode grid fills
// the GPU poorly or K is long.  Measured on MI355X (m = 33 / 64, us, decode
// kernel against 64-row prefill tiles): QKV 10240 x 8192 (decode grid 160 of
// 256 CUs) 30.0 / 35.6 against 24.4 / 28.9 at S = 6; N = 8200, K = 8192 (130
// CUs) 28.9 / 34.6 against 22.1 / 25.7; down 8192 x 28672 57.1 / 62.2
// against 47.1 / 51.2 at S = 8; O 8192 x 8192 (256 CUs, K 8192) keeps the
// decode kernel, 20.6 / 25.5 against 21.7 / 26.5.  Returns the split S (the
// most workgroups that still fit one round, at most 8), or 0 for the decode
// kernel.
static int mid_m_prefill_split(const DecodeShape& d, int64_t K, int NT, int SB) {
    const int64_t wgs = (int64_t)((NT + d.tn * d.nwn - 1) / (d.tn * d.nwn)) * d.s;
    const int64_t rounds = (wgs + kCUs - 1) / kCUs;
    if (4 * wgs >= 3 * rounds * kCUs && K <= 16384) return 0;
    const int NG = (NT + 15) / 16;
    int S = 1;
    while (S < 8 && S < SB && (int64_t)NG * (S + 1) <= kCUs) ++S;
    return S;
}

// The kernel, shape and K split chosen for one problem, and its workspace.
struct GemmPlan {
    enum Kind { kDecode, kPrefill, kPrefillMid } kind;
    int MB;             // decode: 16-row activation blocks
    DecodeShape d;      // decode shape and split
    PrefillShape t;     // prefill shape and split
    size_t ws_bytes;    // workspace fp4_gemm needs
};

static GemmPlan make_plan(int fmt, int64_t M, int64_t N, int64_t K) {
    const int SB = int(padded_k(K) / kScaleBlockK), NT = int(padded_n(N) / kTileN);
    GemmPlan p{};
    if (wide_mid_m(M, NT)) {  // whole-K prefill tiles, no split
        p.kind = GemmPlan::kPrefillMid;
        p.t = PrefillShape{1, 8, 4, 2, 1};
        p.ws_bytes = 0;
    } else if (M <= 64) {
        p.kind = GemmPlan::kDecode;
        p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        p.d = pick_decode(fmt, p.MB, M, N, NT, SB);
        p.ws_bytes = decode_workspace_bytes(p.d, M, N, NT);
        const int S = p.MB == 4 && decode_override().tn == 0 ? mid_m_prefill_split(p.d, K, NT, SB) : 0;
        if (S > 0) {
            p.kind = GemmPlan::kPrefill;
            p.t = PrefillShape{1, 8, 4, 2, S};
            p.ws_bytes = S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
        }
    } else {
        p.kind = GemmPlan::kPrefill;
        p.t = pick_prefill(fmt, M, N, NT, SB);
        p.ws_bytes = p.t.s > 1 ? (size_t)p.t.s * (size_t)M * (size_t)N * sizeof(float) : 0;
    }
    return p;
}

// Plans of recent problems, keyed by (m, N, K, format): a small direct-mapped
// table behind a mutex, so a caller that repeats shapes (every decode step)
// does not rerun the shape models.  No allocation after the first call.
static GemmPlan cached_plan(int fmt, int64_t M, int64_t N, int64_t K) {
    struct Entry {
        int64_t m, n, k;
        int fmt;
        bool used;
        GemmPlan plan;
    };
    constexpr int kEntries = 64;
    static Entry table[kEntries];
    static std::mutex mu;
    const uint64_t h = ((uint64_t)M * 0x9E3779B97F4A7C15ull) ^ ((uint64_t)N * 0xC2B2AE3D27D4EB4Full) ^
                       ((uint64_t)K * 0x165667B19E3779F9ull) ^ (uint64_t)fmt;
    Entry& e = table[(h >> 32) % kEntries];
    {
        std::lock_guard<std::mutex> lock(mu);
        if (e.used && e.m == M && e.n == N && e.k == K && e.fmt == fmt) return e.plan;
    }
    const GemmPlan plan = make_plan(fmt, M, N, K);
    std::lock_guard<std::mutex> lock(mu);
    e = Entry{M, N, K, fmt, true, plan};
    return plan;
}

static int launch_gemm(const GemmPlan& plan, int fmt, int act, const void* A, const void* wq, const void* sq,
                       void* C, void* ws, int M, int N, int K, int KB, int SB, int NT, float alpha, hipStream_t s) {
    if (plan.kind == GemmPlan::kPrefillMid) {
        const bool ok = act == 0 ? launch_prefill_bf16(fmt, plan.t, A, wq, sq, C, nullptr, M, N, K, KB, SB, NT, alpha, s)
                                 : launch_prefill_f16(fmt, plan.t, A, wq, sq, C, nullptr, M, N, K, KB, SB, NT, alpha, s);
        return ok ? FP4_OK : FP4_ERR_SHAPE;
    }
    if (plan.kind == GemmPlan::kDecode) {
        const DecodeShape& d = plan.d;
        float* P = d.s > 1 ? static_cast<float*>(ws) : nullptr;
        const uint32_t tag = P ? next_split_tag() : 0u;
        const bool ok =
            act == 0 ? launch_decode_bf16(fmt, plan.MB, d, A, wq, sq, C, P, M, N, K, KB, SB, NT, alpha, tag, s)
                     : launch_decode_f16(fmt, plan.MB, d, A, wq, sq, C, P, M, N, K, KB, SB, NT, alpha, tag, s);
        return ok ? FP4_OK : FP4_ERR_SHAPE;
    }
    const PrefillShape& t = plan.t;
    float* P = t.s > 1 ? static_cast<float*>(ws) : nullptr;
    const bool ok = act == 0 ? launch_prefill_bf16(fmt, t, A, wq, sq, C, P, M, N, K, KB, SB, NT, alpha, s)
                             : launch_prefill_f16(fmt, t, A, wq, sq, C, P, M, N, K, KB, SB, NT, alpha, s);
    if (!ok) return FP4_ERR_SHAPE;
    if (P) launch_reduce(act, P, C, (int64_t)M * N, t.s, alpha, s);
    return FP4_OK;
}

// Workspace bytes of the kernel fp4_gemm picks for this problem.
static size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
    if (M == 0) return 0;
    return cached_plan(fmt, M, N, K).ws_bytes;
}

// alpha: finite, |alpha| in [2^-100, 2^100] or exactly 1 (checked by the entries).
static bool alpha_ok(float alpha) {
    const float a = fabsf(alpha);
    return a == 1.0f || (a >= 0x1p-100f && a <= 0x1p100f);
}

// Scratch of fp4_gemm_noalloc: the split-K partial sums and arrival words
// that fp4_gemm keeps in the caller's workspace, in a file-scope device
// array instead.  Every GPU the library runs on holds its own copy until the
// process ends; host code never uses the array's name as an address, only
// the per-device pointer hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];  // per device id, set once with that device current

// The current device's address of `scratch` (looked up on the first call on
// each device).
static int noalloc_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP4_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP4_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FP4_OK;
}

// use_scratch: fp4_gemm_noalloc (workspace arguments ignored; the device's
// `scratch` array serves as the workspace, FP4_ERR_WORKSPACE beyond its size).
static int gemm_impl(int act, const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N,
                     int64_t K, int format, float alpha, void* workspace, size_t workspace_bytes, void* stream,
                     bool use_scratch = false) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (act != 0 && act != 1) return FP4_ERR_FORMAT;
    if (!alpha_ok(alpha)) return FP4_ERR_VALUE;
    if (m < 0 || m > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    if (m == 0) return FP4_OK;
    if (!A || !wq || !sq || !C) return FP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(sq) |
         reinterpret_cast<uintptr_t>(C)) & 15)
        return FP4_ERR_SHAPE;
    if (round_up(m, a_row_block(m)) * K * 2 >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
    if (m * N * 2 >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;  // Y through 32-bit ranged offsets
    const GemmPlan plan = cached_plan(format, m, N, K);
    const size_t need = plan.ws_bytes;
    if (use_scratch) {
        if (need > kNoAllocScratchBytes) return FP4_ERR_WORKSPACE;
    } else if (need > 0 &&
               (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15))) {
        return FP4_ERR_WORKSPACE;
    }
    st = check_device();
    if (st != FP4_OK) return st;
    if (use_scratch && need > 0) {
        st = noalloc_scratch(&workspace);
        if (st != FP4_OK) return st;
    }
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int KB = int(Kp / kChunkK), SB = int(Kp / kScaleBlockK), NT = int(Np / kTileN);
    (void)hipGetLastError();
    st = launch_gemm(plan, format, act, A, wq, sq, C, workspace, int(m), int(N), int(K), KB, SB, NT, alpha,
                     reinterpret_cast<hipStream_t>(stream));
    if (st != FP4_OK) return st;
    return launch_status();
}

static int dequant_impl(int act, const void* wq, const void* sq, void* W, int64_t N, int64_t K, int format,
                        void* stream) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (!wq || !sq || !W) return FP4_ERR_NULL;
    st = check_device();
    if (st != FP4_OK) return st;
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int KB = int(Kp / kChunkK), SB = int(Kp / kScaleBlockK), NT = int(Np / kTileN);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const dim3 grid(NT, KB), block(64);
    const u32x4* q = (const u32x4*)wq;
    const uint8_t* sc = (const uint8_t*)sq;
    uint16_t* o = (uint16_t*)W;
    if (format == FP4_NVFP4 && act == 0) dequant_kernel<0, 0><<<grid, block, 0, s>>>(q, sc, o, int(N), int(K), KB, SB);
    if (format == FP4_NVFP4 && act == 1) dequant_kernel<0, 1><<<grid, block, 0, s>>>(q, sc, o, int(N), int(K), KB, SB);
    if (format == FP4_MXFP4 && act == 0) dequant_kernel<1, 0><<<grid, block, 0, s>>>(q, sc, o, int(N), int(K), KB, SB);
    if (format == FP4_MXFP4 && act == 1) dequant_kernel<1, 1><<<grid, block, 0, s>>>(q, sc, o, int(N), int(K), KB, SB);
    return launch_status();
}

// Grouped MoE GEMM.  The row counts per expert live on the device, so the
// grid is sized for the worst case (sum over experts of ceil(rows / block)
// <= P / block + E row blocks) and surplus workgroups exit at once.  Row
// block: 16 rows while the mean rows per expert is at most 16, else 32 or
// 64.  Tiles per workgroup: the most (16, 8, 4, 2) that still give about
// 1024 workgroups over the likely row blocks (min(P, E) for one-row-block
// experts): an active expert's weights are streamed once per row block, so
// the grid should cover the CUs several times over.
static int moe_impl(const void* A, const void* wq, const void* sq, const int32_t* ids, const int32_t* offsets,
                    const float* topw, void* C, int64_t a_rows, int64_t a_div, int64_t out_rows, int64_t P,
                    int64_t E, int64_t N, int64_t K, int format, void* stream) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (E < 1 || E > 4096 || P < 0 || P > (int64_t(1) << 24) || a_div < 1 || a_rows < 1 || out_rows < 1 ||
        out_rows > (int64_t(1) << 24))
        return FP4_ERR_SHAPE;
    if (P == 0) return FP4_OK;
    if (!A || !wq || !sq || !ids || !offsets || !C) return FP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(sq) |
         reinterpret_cast<uintptr_t>(C)) & 15)
        return FP4_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(ids) | reinterpret_cast<uintptr_t>(offsets) |
         reinterpret_cast<uintptr_t>(topw)) & 3)
        return FP4_ERR_SHAPE;
    if (round_up(a_rows, 64) * K * 2 >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
    if (out_rows * N * 2 >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;  // C through 32-bit ranged offsets
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int KB = int(Kp / kChunkK), SB = int(Kp / kScaleBlockK), NT = int(Np / kTileN);
    const int64_t G = format == FP4_NVFP4 ? 16 : 32;
    const int64_t w_stride = Np * Kp / 2, s_stride = Np * Kp / G;
    const int64_t mean_rows = (P + E - 1) / E;
    const int MB = mean_rows <= 16 ? 1 : (mean_rows <= 32 ? 2 : 4);
    const int64_t rows = 16 * MB;
    const int64_t items = (P + rows - 1) / rows + E;
    if (items > 65535) return FP4_ERR_SHAPE;
    st = check_device();
    if (st != FP4_OK) return st;
    const int64_t likely = std::max<int64_t>(1, std::min(P, E));
    static const int kTw[4][3] = {{16, 2, 8}, {8, 1, 8}, {4, 1, 4}, {2, 1, 2}};
    int pick = 3;
    for (int i = 0; i < 4; ++i)
        if (likely * ((NT + kTw[i][0] - 1) / kTw[i][0]) >= 1024) {
            pick = i;
            break;
        }
    int tn = kTw[pick][1], nwn = kTw[pick][2];
    if (MB > 1 && tn * nwn == 2) nwn = 4;  // the two-tile shape is compiled for 16-row blocks only
    MoeArgs moe{ids, offsets, topw, int(E), int(P), int(a_div), int(a_rows), int(out_rows), w_stride, s_stride};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (!launch_moe_bf16(format, MB, tn, nwn, A, wq, sq, C, moe, int(N), int(K), KB, SB, NT, int(items), s))
        return FP4_ERR_SHAPE;
    return launch_status();
}

// Largest number of G-element blocks one quantizer launch covers (one thread
// each, so far below the 2^32 work-items a dispatch can count).
constexpr int64_t kQuantSliceGroups = int64_t(1) << 26;

static int quantize_impl(const void* W, void* codes, void* scales, int64_t N, int64_t K, int format, float alpha,
                         void* stream) {
    if (format != FP4_NVFP4 && format != FP4_MXFP4) return FP4_ERR_FORMAT;
    const int64_t G = format == FP4_NVFP4 ? 16 : 32;
    if (N < 1 || K < G || K % G || N > (int64_t(1) << 24) || K > (int64_t(1) << 24)) return FP4_ERR_SHAPE;
    if (!W || !codes || !scales) return FP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(W) & 15) || (reinterpret_cast<uintptr_t>(codes) & (G / 2 - 1)))
        return FP4_ERR_SHAPE;
    if (!(alpha > 0.0f) || !alpha_ok(alpha)) return FP4_ERR_VALUE;
    int st = check_device();
    if (st != FP4_OK) return st;
    // One thread per G-element block.  A dispatch counts its work-items in 32
    // bits, so the rows go out in slices of at most kQuantSliceGroups blocks
    // (whole rows; a row has at most 2^20 blocks).
    const int64_t gpr = K / G;
    const int64_t rows_per = std::max<int64_t>(1, kQuantSliceGroups / gpr);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    for (int64_t r0 = 0; r0 < N; r0 += rows_per) {
        const int64_t groups = std::min(rows_per, N - r0) * gpr;
        const uint16_t* w = static_cast<const uint16_t*>(W) + r0 * K;
        uint8_t* c = static_cast<uint8_t*>(codes) + r0 * (K / 2);
        uint8_t* sc = static_cast<uint8_t*>(scales) + r0 * gpr;
        const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
        if (format == FP4_NVFP4)
            quantize_kernel<0><<<grid, block, 0, s>>>(w, c, sc, groups, alpha, gpr, gpr);
        else
            quantize_kernel<1><<<grid, block, 0, s>>>(w, c, sc, groups, alpha, gpr, gpr);
        st = launch_status();
        if (st != FP4_OK) return st;
    }
    return FP4_OK;
}

// Native FP4 path: workspace = quantized activations (m rows of Kp / 2 code
// bytes, then m rows of Kp / 32 scale bytes, 256-byte aligned) + FP32
// partials of a K split.  K split: the largest S <= 8 (and <= Kp / 512) that
// keeps blocks * S within one round of 256 workgroups.
// Native kernel shape: four waves of 4 m-blocks x 2 n-tiles (BM 64, BN 128;
// 357 VGPRs).  Eight m-blocks per wave do not fit the registers.
static int native_bm() { return 64; }
static int native_bnt() { return 8; }

struct NativePlan {
    int64_t codes_bytes, scales_off, scales_bytes, partial_off;
    int S;
    size_t total;
};
static NativePlan native_plan(int64_t m, int64_t N, int64_t K) {
    NativePlan p{};
    const int64_t Kp = padded_k(K), QB = Kp / kScaleBlockK, NT = padded_n(N) / kTileN;
    p.codes_bytes = m * Kp / 2;
    p.scales_off = round_up(p.codes_bytes, 256);
    p.scales_bytes = m * Kp / 32;
    p.partial_off = round_up(p.scales_off + p.scales_bytes, 256);
    const int64_t blocks = ((m + native_bm() - 1) / native_bm()) * ((NT + native_bnt() - 1) / native_bnt());
    p.S = 1;
    while (p.S < 8 && 2 * p.S <= QB && blocks * 2 * p.S <= kCUs && m * N < (int64_t(1) << 29)) p.S *= 2;
    p.total = size_t(p.partial_off) + (p.S > 1 ? size_t(p.S) * size_t(m) * size_t(N) * 4 : 0);
    return p;
}

static int native_check(int64_t m, int64_t N, int64_t K) {
    int st = fp4_check_weight_shape(N, K, FP4_MXFP4);
    if (st != FP4_OK) return st;
    if (m < 0 || m > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    if (round_up(m, 128) * padded_k(K) / 2 >= (int64_t(1) << 31) || round_up(m, 128) * N * 2 >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    return FP4_OK;
}

static int native_impl(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                       float alpha, void* workspace, size_t workspace_bytes, void* stream) {
    int st = native_check(m, N, K);
    if (st != FP4_OK) return st;
    if (!alpha_ok(alpha)) return FP4_ERR_VALUE;
    if (m == 0) return FP4_OK;
    if (!A || !wq || !sq || !C) return FP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(sq) |
         reinterpret_cast<uintptr_t>(C)) & 15)
        return FP4_ERR_SHAPE;
    const NativePlan p = native_plan(m, N, K);
    if (!workspace || workspace_bytes < p.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
        return FP4_ERR_WORKSPACE;
    st = check_device();
    if (st != FP4_OK) return st;
    const int64_t Kp = padded_k(K), Np = padded_n(N);
    const int KB = int(Kp / kChunkK), NT = int(Np / kTileN);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* aq = ws;
    uint8_t* as = ws + p.scales_off;
    float* P = p.S > 1 ? reinterpret_cast<float*>(ws + p.partial_off) : nullptr;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int64_t groups = m * (Kp / 32);
    quantize_kernel<1><<<dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s>>>(
        (const uint16_t*)A, aq, as, groups, 1.0f, K / 32, Kp / 32);
    const int MT = int((m + native_bm() - 1) / native_bm()), NG = (NT + native_bnt() - 1) / native_bnt();
    const dim3 grid(MT * NG * p.S), block(256);
    gemm_native<1, 4, 4, 2><<<grid, block, 0, s>>>(aq, as, (const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)C, P,
                                                   int(m), int(N), KB, NT, p.S, alpha);
    if (P) launch_reduce(0, P, C, m * N, p.S, alpha, s);
    return launch_status();
}

}  // namespace fp4

using namespace fp4;

extern "C" int fp4_gemm_native_workspace_size(int64_t m, int64_t N, int64_t K, size_t* bytes) {
    int st = native_check(m, N, K);
    if (st != FP4_OK) return st;
    if (!bytes) return FP4_ERR_NULL;
    *bytes = m == 0 ? 0 : native_plan(m, N, K).total;
    return FP4_OK;
}

extern "C" int fp4_gemm_native(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                               float alpha, void* workspace, size_t workspace_bytes, void* stream) {
    return native_impl(A, wq, sq, C, m, N, K, alpha, workspace, workspace_bytes, stream);
}

extern "C" int fp4_gemm_ex(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                           int format, int act_type, float alpha, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return gemm_impl(act_type, A, wq, sq, C, m, N, K, format, alpha, workspace, workspace_bytes, stream);
}

extern "C" int fp4_quantize(const void* W, void* codes, void* scales, int64_t N, int64_t K, int format, float alpha,
                            void* stream) {
    return quantize_impl(W, codes, scales, N, K, format, alpha, stream);
}

extern "C" int fp4_moe_gemm(const void* A, const void* wq, const void* sq, const int32_t* sorted_ids,
                            const int32_t* expert_offsets, const float* topk_weights, void* C, int64_t a_rows,
                            int64_t a_div, int64_t out_rows, int64_t P, int64_t E, int64_t N, int64_t K, int format,
                            void* stream) {
    return moe_impl(A, wq, sq, sorted_ids, expert_offsets, topk_weights, C, a_rows, a_div, out_rows, P, E, N, K,
                    format, stream);
}

extern "C" int fp4_gemm_workspace_size(int64_t m, int64_t N, int64_t K, int format, size_t* bytes) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (m < 0 || m > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    if (!bytes) return FP4_ERR_NULL;
    *bytes = gemm_workspace_bytes(m, N, K, format);
    return FP4_OK;
}

extern "C" int fp4_gemm(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                        int format, void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_impl(0, A, wq, sq, C, m, N, K, format, 1.0f, workspace, workspace_bytes, stream);
}

extern "C" int fp4_gemm_noalloc(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N,
                                int64_t K, int format, void* stream) {
    return gemm_impl(0, A, wq, sq, C, m, N, K, format, 1.0f, nullptr, 0, stream, true);
}

extern "C" size_t fp4_gemm_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

extern "C" int fp4_gemm_f16(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                            int format, void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_impl(1, A, wq, sq, C, m, N, K, format, 1.0f, workspace, workspace_bytes, stream);
}

extern "C" int fp4_dequant(const void* wq, const void* sq, void* W_bf16, int64_t N, int64_t K, int format,
                           void* stream) {
    return dequant_impl(0, wq, sq, W_bf16, N, K, format, stream);
}

extern "C" int fp4_dequant_f16(const void* wq, const void* sq, void* W_f16, int64_t N, int64_t K, int format,
                               void* stream) {
    return dequant_impl(1, wq, sq, W_f16, N, K, format, stream);
}
