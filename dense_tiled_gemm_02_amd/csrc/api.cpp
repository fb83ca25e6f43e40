// C ABI of the tiled GEMM library: validation, planner (tile-configuration
// choice), plan cache and launch.  Declarations and the contract of every
// entry point are in include/gemm.h.
//
// The planner keys its choice on every dimension the kernels tile on
// (M, N, K), the storage type, the layout and the presence of C ("Tuning
// Triton", section 3: a cache key that omits a tiled dimension silently serves
// a wrong tile), and separates regimes (section 4: a skinny M wants a
// different tile family from a square problem).  It prunes by the LDS budget
// of the device (FlagGems "Hygon optimization", section "Software
// pipelining": stages x (BLOCK_M + BLOCK_N) x BLOCK_K x 2 bytes).

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <cstdlib>
#include <vector>

#include "../../include/gemm.h"
#include "api_internal.h"
#include "kernels.h"
#include "tile_order.h"

struct gemm_plan {
    gemm_problem prob;
    gemm_problem view;                  // the problem in the kernels' units (int8: pairs of k)
    gemm_device_info dev;
    gemm_config cfg;
    const dtg::KernelEntry* entry;      // the chosen variant
    const dtg::KernelEntry* fallback;   // element-wise variant, for unaligned bases
    int64_t num_pid_m, num_pid_n, grid;
    int64_t ws_bytes;                   // workspace the chosen kernel needs
};

namespace {

thread_local std::string g_err;

gemm_status fail(gemm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gemm_status fail(gemm_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

gemm_status ok() { return GEMM_OK; }

bool log_enabled() {
    static const bool on = [] {
        const char* v = getenv("GEMM_LOG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

gemm_status validate(const gemm_problem* p) {
    if (!p) return fail(GEMM_ERR_INVALID_ARG, "problem is NULL");
    if (p->M < 0 || p->N < 0 || p->K < 0)
        return fail(GEMM_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld", (long long)p->M,
                    (long long)p->N, (long long)p->K);
    if (p->dtype != GEMM_F16 && p->dtype != GEMM_BF16 && p->dtype != GEMM_I8)
        return fail(GEMM_ERR_INVALID_ARG, "dtype %d is none of GEMM_F16, GEMM_BF16, GEMM_I8", (int)p->dtype);
    if (p->has_c != 0 && p->has_c != 1)
        return fail(GEMM_ERR_INVALID_ARG, "has_c must be 0 or 1, got %d", (int)p->has_c);
    if (p->M > kMaxDim || p->N > kMaxDim || p->K > kMaxDim)
        return fail(GEMM_ERR_UNSUPPORTED, "dimensions above 2^31-1 are not supported");
    const int64_t rs[4] = {p->sa_m, p->sb_k, p->sc_m, p->sd_m};
    const int64_t cs[4] = {p->sa_k, p->sb_n, p->sc_n, p->sd_n};
    const char* nm[4] = {"A", "B", "C", "D"};
    for (int i = 0; i < 4; ++i) {
        if (i == 2 && !p->has_c) continue;
        if (rs[i] < 0 || cs[i] < 0)
            return fail(GEMM_ERR_UNSUPPORTED, "negative stride of %s", nm[i]);
        const int64_t rows = (i == 0) ? p->M : (i == 1) ? p->K : p->M;
        const int64_t cols = (i == 0) ? p->K : p->N;
        if (rows == 0 || cols == 0) continue;
        if (i >= 2 && cs[i] != 1 && cols > 1)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "%s column stride %lld: C and D must be row-major (column stride 1)",
                        nm[i], (long long)cs[i]);
        if (i == 3 && rows > 1 && rs[i] < cols)
            return fail(GEMM_ERR_INVALID_ARG, "D row stride %lld < N=%lld makes output rows overlap",
                        (long long)rs[i], (long long)cols);
    }
    const int64_t pm = (p->M + 15) / 16, pn = (p->N + 15) / 16;
    if (pm * pn > kMaxDim) return fail(GEMM_ERR_UNSUPPORTED, "output too large for one launch");
    return ok();
}

// How A and B sit in memory: 0 (both row-major), dtg::kLayTA (A stored
// K x M: unit m stride), dtg::kLayTB (B stored N x K: unit k stride), both, or
// -1 (any other strides: element-wise path only).  A single row or column
// counts as row-major.
int layout_of(const gemm_problem* p) {
    const bool a_rm = p->K <= 1 || p->sa_k == 1;
    const bool a_cm = !a_rm && (p->M <= 1 || p->sa_m == 1);
    const bool b_rm = p->N <= 1 || p->sb_n == 1;
    const bool b_cm = !b_rm && (p->K <= 1 || p->sb_k == 1);
    if ((!a_rm && !a_cm) || (!b_rm && !b_cm)) return -1;
    return (a_cm ? dtg::kLayTA : 0) | (b_cm ? dtg::kLayTB : 0);
}

// The operand layout the kernels take a problem in: int8 operands are always
// A row-major and B stored N x K (k contiguous), also when a single row or
// column would read as either.
int kernel_layout(const gemm_problem* p) { return p->dtype == GEMM_I8 ? dtg::kLayTB : layout_of(p); }

// The problem in the units the tile kernels address: for GEMM_I8 one unit is
// a pair of int8 along k (K and the leading strides of A and B halved; C and
// D keep their int32 strides); otherwise the problem itself.
// GEMM_ERR_UNSUPPORTED for int8 operands the kernels cannot take.
gemm_status kernel_view(const gemm_problem* p, gemm_problem* v) {
    *v = *p;
    if (p->dtype != GEMM_I8 || p->K == 0) return GEMM_OK;
    const bool a_ok = (p->K <= 1 || p->sa_k == 1) && (p->M <= 1 || p->sa_m % 16 == 0);
    const bool b_ok = (p->K <= 1 || p->sb_k == 1) && (p->N <= 1 || p->sb_n % 16 == 0);
    if (p->K % 16 != 0 || !a_ok || !b_ok)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "int8 operands must have k contiguous (A row-major, B stored N x K), K and their leading "
                    "strides multiples of 16 (K=%lld, A strides %lld,%lld, B strides %lld,%lld)",
                    (long long)p->K, (long long)p->sa_m, (long long)p->sa_k, (long long)p->sb_k,
                    (long long)p->sb_n);
    v->K = p->K / 2;
    v->sa_k = 1;
    v->sa_m = p->M > 1 ? p->sa_m / 2 : v->K;
    v->sb_k = 1;
    v->sb_n = p->N > 1 ? p->sb_n / 2 : v->K;
    return GEMM_OK;
}

// The 16-byte vector paths move 8 elements along each operand's contiguous
// index: that index's extent and the other stride must be multiples of 8.
bool vec_shape_ok(const gemm_problem* p) {
    const int lay = kernel_layout(p);
    if (lay < 0) return false;
    const bool a_ok = (lay & dtg::kLayTA) ? (p->M % 8 == 0 && p->sa_k % 8 == 0)
                                          : (p->K % 8 == 0 && p->sa_m % 8 == 0);
    const bool b_ok = (lay & dtg::kLayTB) ? (p->K % 8 == 0 && p->sb_n % 8 == 0)
                                          : (p->N % 8 == 0 && p->sb_k % 8 == 0);
    return a_ok && b_ok;
}

// The direct-to-LDS kernels address one BM-row panel of A and one BK-row slab
// of B with 32-bit byte offsets from descriptors rebased every K step, and
// rely on the descriptor's range to zero the rows past K of an operand kept
// as rows of k (A stored K x M, row-major B): that needs its row stride to be
// at least its contiguous extent (M or N), else the element-wise path runs.
bool dma_offsets_ok(const gemm_problem* p, const dtg::KernelEntry* e) {
    const int64_t lim = (int64_t(1) << 31) - 4096;
    const bool ta = e->layout > 0 && (e->layout & dtg::kLayTA), tb = e->layout > 0 && (e->layout & dtg::kLayTB);
    const int64_t a = ta ? static_cast<int64_t>(e->bk) * p->sa_k * 2 + e->bm * 2
                         : static_cast<int64_t>(e->bm) * p->sa_m * 2 + e->bk * 2;
    const int64_t b = tb ? static_cast<int64_t>(e->bn) * p->sb_n * 2 + e->bk * 2
                         : static_cast<int64_t>(e->bk) * p->sb_k * 2 + e->bn * 2;
    if (ta && p->K > 1 && p->sa_k < p->M) return false;
    if (!tb && p->K > 1 && p->sb_k < p->N) return false;
    return a < lim && b < lim;
}

// The skinny kernels address a CK-row chunk of B (and of A's rows) with
// 32-bit byte offsets from a descriptor rebased at every chunk: row r of the
// chunk, column c at r * ldb * 2 + c * 2 (A: row i at i * lda * 2 + k * 2).
// Beyond the descriptor range cap the loads would read zeros, so such strides
// go to another kernel.
bool skinny_offsets_ok(const gemm_problem* p, const dtg::KernelEntry* e) {
    const int64_t lim = (int64_t(1) << 31) - 4096;
    const int64_t b = static_cast<int64_t>(e->bk) * p->sb_k * 2 + p->N * 2 + 256;
    const int64_t a = static_cast<int64_t>(e->bm) * p->sa_m * 2 + static_cast<int64_t>(e->bk) * 2 + 256;
    return a < lim && b < lim;
}

std::vector<const dtg::KernelEntry*> all_entries() {
    std::vector<const dtg::KernelEntry*> v;
    int n = 0;
    const dtg::KernelEntry* t = dtg::tile_kernel_table(&n);
    for (int i = 0; i < n; ++i) v.push_back(&t[i]);
    t = dtg::dma_kernel_table(&n);
    for (int i = 0; i < n; ++i) v.push_back(&t[i]);
    t = dtg::i8_kernel_table(&n);
    for (int i = 0; i < n; ++i) v.push_back(&t[i]);
    t = dtg::skinny_kernel_table(&n);
    for (int i = 0; i < n; ++i) v.push_back(&t[i]);
    return v;
}

bool matches(const dtg::KernelEntry* e, const gemm_config& f) {
    return (f.kernel == 0 || f.kernel == e->family) && (f.bm == 0 || f.bm == e->bm) &&
           (f.bn == 0 || f.bn == e->bn) && (f.bk == 0 || f.bk == e->bk) &&
           (f.stages == 0 || f.stages == e->stages) && (f.mfma == 0 || f.mfma == e->mfma) &&
           (f.waves_m == 0 || f.waves_m == e->waves_m) && (f.waves_n == 0 || f.waves_n == e->waves_n) &&
           (f.splitk <= 1 || e->splitk == 0 || f.splitk <= e->splitk);   // e->splitk: most slices, 0 = any
}

// The first compiled variant that fits the device and the problem's layout
// and matches `want`.
const dtg::KernelEntry* find_entry(const gemm_config& want, int dtype, int vec,
                                   const gemm_device_info& dev, const gemm_problem* p) {
    const int lay = kernel_layout(p);
    for (const dtg::KernelEntry* e : all_entries()) {
        if (e->dtype != dtype || e->vec != vec || e->stream_b) continue;   // streamed-B twins: stream_b_twin
        if (e->layout != -1 && e->layout != lay) continue;
        if (e->lds_bytes > dev.lds_per_wg) continue;
        if ((e->family == dtg::KF_DMA || e->family == dtg::KF_DMA_SK) && !dma_offsets_ok(p, e)) continue;
        if (e->family == dtg::KF_SKINNY && !skinny_offsets_ok(p, e)) continue;
        if (matches(e, want)) return e;
    }
    return nullptr;
}

// The streamed-B twin of a direct-to-LDS variant (the same tile, ring, waves
// and layout; B loaded non-temporal), or e itself when there is none.  Taken
// when the grid has one row of tiles, so every byte of B is read once per K
// slice and caching it gains nothing.
const dtg::KernelEntry* stream_b_twin(const dtg::KernelEntry* e, const gemm_device_info& dev,
                                      const gemm_problem* p) {
    for (const dtg::KernelEntry* t : all_entries()) {
        if (t->stream_b && t->family == e->family && t->bm == e->bm && t->bn == e->bn && t->bk == e->bk &&
            t->stages == e->stages && t->mfma == e->mfma && t->waves_m == e->waves_m && t->waves_n == e->waves_n &&
            t->dtype == e->dtype && t->vec == e->vec && t->layout == e->layout && t->lds_bytes <= dev.lds_per_wg &&
            dma_offsets_ok(p, t))
            return t;
    }
    return e;
}

gemm_config cfg_of(int fam, int bm, int bn, int bk, int st, int mf, int wm, int wn) {
    gemm_config c;
    memset(&c, 0, sizeof c);
    c.kernel = fam; c.bm = bm; c.bn = bn; c.bk = bk; c.stages = st; c.mfma = mf;
    c.waves_m = wm; c.waves_n = wn; c.splitk = 1;
    return c;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Measured choices for exact problem keys (M, N, K, dtype, has_c; row-major
// operands on the vector path), the winners of the interleaved races of
// dense_tiled_gemm_02_amd/tune.py (a pruned sweep, every candidate probed in
// its own process; a winner must beat the heuristic's plan beyond the
// noise), frozen into tuned_table.inc.  Anything not listed, or listed with
// a configuration this device cannot run, takes the regime heuristic below.
struct TunedKey {
    int64_t M, N, K;
    int dtype, has_c;
    gemm_config cfg;
    int group_m, xcd;
};
const std::vector<TunedKey>& tuned_table() {
    static const std::vector<TunedKey> t = {
#include "tuned_table.inc"
    };
    // GEMM_TUNED_TABLE=0 plans every shape by the heuristic alone (a re-tune
    // races the candidates against the heuristic, not against the old table)
    static const std::vector<TunedKey> none;
    static const bool off = [] {
        const char* v = std::getenv("GEMM_TUNED_TABLE");
        return v && v[0] == '0';
    }();
    return off ? none : t;
}

// Regime heuristic.  Square / tail problems take the largest tile that still
// gives every CU at least one workgroup; skinny M takes a short-M tile.
gemm_config heuristic(const gemm_problem* p, const gemm_device_info& dev, int* group_m, bool allow_ws) {
    const int64_t M = p->M, N = p->N, K = p->K;
    *group_m = 8;
    if (M <= 32 && kernel_layout(p) == 0) {
        // Decode regime, bucketed by M: 16-row slabs for M <= 16, 32-row slabs
        // (two MFMA row blocks) for M <= 32.  Stream B: each workgroup reads a
        // band of every row of its K slice, and the slices supply the
        // workgroups (one per CU: these kernels hold most of the LDS).  The
        // slab is the widest of 128, 64 and 32 columns (256-, 128- and 64-byte
        // bands) whose slabs fill the CUs with 4 K slices, then S = CUs /
        // slabs, at most 8, each slice >= 512 k.  Four slices is where the
        // per-slice exchange and the streaming balance: swept at M in {1, 4,
        // 16, 32} x N = K in {2048, 4096, 8192} (bf16, every compiled decode
        // variant, interleaved races), the winners at M <= 16 are 128-column
        // slabs with 4 slices at 8192 (29.2 us), 64-column slabs of 4 waves with
        // 4 slices at 4096 (11.4 us; 128 columns with 8 slices 12.2 us) and
        // 32-column slabs with 4 slices at 2048 (6.8-7.0 us; 128 columns with
        // 4 slices, i.e. a quarter of the CUs, 8.1-8.8 us).  When 128-column
        // slabs fill the CUs with up to 8 slices of at least 512 k each, they
        // beat the narrower slabs of the 4-slice rule: at first for a long K
        // (N = 4096, K = 11008: 20.4 against 22.5 us; K = 14336: 26.4 against
        // 28.1 us, at M = 1 and 16), and since the wide slabs walk their chunks
        // rotated and stream B non-temporal, at N = K = 4096 too (M = 1, 4, 16:
        // 11.0-11.2 against 11.2-11.5 us).  The 32-row slabs keep 1024 k: at
        // M = 32, N = K = 4096, 128 columns with 8 slices take 14.6 us against
        // 12.6 for the 4-slice rule's 64 columns.
        if (allow_ws && cdiv(N, 128) <= 4096) {
            const int64_t s_max = K / 512 < 4 ? (K / 512 > 1 ? K / 512 : 1) : 4;
            int bn = 32;
            for (int w : {128, 64}) {
                if (cdiv(N, w) * s_max >= dev.cu_count) {
                    bn = w;
                    break;
                }
            }
            if (bn < 128) {
                int64_t s128 = dev.cu_count / cdiv(N, 128);
                if (s128 > 8) s128 = 8;
                if (cdiv(N, 128) * s128 >= dev.cu_count && K / s128 >= (M <= 16 ? 512 : 1024)) bn = 128;
            }
            const int64_t slabs = cdiv(N, bn);
            int64_t s = dev.cu_count / (slabs > 0 ? slabs : 1);
            if (s > 8) s = 8;
            while (s > 1 && K / s < 512) --s;
            if (s < 1) s = 1;
            const int bm = M <= 16 ? 16 : 32;
            gemm_config c = bn == 128  ? cfg_of(dtg::KF_SKINNY, bm, 128, 32, 2, 16, 1, 8)
                            : bn == 64 ? cfg_of(dtg::KF_SKINNY, bm, 64, bm == 16 ? 64 : 32, 3, 16, 1, bm == 16 ? 4 : 8)
                                       : cfg_of(dtg::KF_SKINNY, bm, 32, bm == 16 ? 64 : 32, 3, 16, 1, 8);
            c.splitk = static_cast<int32_t>(s);
            return c;
        }
        // no workspace: one workgroup per 32-column slab, K split over its 8 waves
        const int bn = (cdiv(N, 32) >= dev.cu_count || M > 16) ? 32 : 16;
        gemm_config c = cfg_of(dtg::KF_SKINNY, M <= 16 ? 16 : 32, bn, M <= 16 ? 64 : 32, 3, 16, 1, 8);
        c.splitk = 1;
        return c;
    }
    // 8-wave direct-to-LDS tiles chosen by estimated time: rounds of
    // workgroups, ceil(tiles / (CUs x workgroups resident per CU)), times the
    // tile's cost per round relative to 256 x 256 (a 1-wave-per-SIMD tile
    // hides far less latency, so the ladder holds 8-wave tiles only).  The
    // mid tiles run 3-stage rings, 128 x 128 a 4-stage ring (one workgroup per
    // CU) or a 2-stage one (64 KiB: two per CU).  Relative costs fitted to
    // forced runs of every candidate at nine shapes (bf16 medians, one box,
    // interleaved): 4096^3 256 x 256 101 us (256 x 128 117, 128 x 128 125),
    // 3072^2 x 4096 256 x 256 82 us (99), 3584^2 x 4096 256 x 256 86 us (102),
    // 2560^2 x 4096 256 x 128 51 us (128 x 128 55, 256 x 256 76), 2048^2 x
    // 4096 128 x 128 / 4 stages 36 us (256 x 128 47, 256 x 256 75), 1536^2 x
    // 8192 128 x 128 / 4 stages 60 us (85), 4096 x 2048 x 8192 256 x 128
    // 111 us (128 x 128 120, 256 x 256 159), 4000 x 3000 x 1000 256 x 256
    // 31 us (128 x 256 36); and for small problems the 4-wave 64 x 64 tile
    // (64 KiB: two per CU) with a 4-stage ring, fp16: 1024^3 8.3 us
    // (128 x 128 11.2), 512^3 5.5 us (7.3), 768^2 x 2048 11.7 us (23.1),
    // 1024^2 x 4096 20.3 us (128 x 128 44.4).  The 192 x 256 tile (compiled
    // for row-major A and B only) covers the band where 256 x 256 tiles leave
    // CUs idle and 256 x 128 tiles need a second round: 3072^2 x 4096 73.3 us
    // (256 x 256 86.5), 4000 x 3000 x 1000 + C 35.2 us (38.7), bitwise the
    // same result; 2560^2 x 4096 66.2 us against 49.6 for 256 x 128.  K
    // slices across workgroups (deterministic fused reduce) replace the
    // ladder where they fit (below).
    struct C { int fam, bm, bn, bk, st, mf, wm, wn, per_cu; double cost; bool row_major_only; };
    static const C ladder[] = {
        {dtg::KF_DMA, 256, 256, 64, 2, 16, 2, 4, 1, 1.0, false},
        {dtg::KF_DMA, 256, 128, 64, 3, 16, 4, 2, 1, 0.64, false},
        {dtg::KF_DMA, 128, 256, 64, 3, 16, 2, 4, 1, 0.64, false},
        {dtg::KF_DMA, 128, 128, 64, 4, 16, 2, 4, 1, 0.43, false},
        {dtg::KF_DMA, 128, 128, 64, 2, 16, 2, 4, 2, 0.68, false},
        {dtg::KF_DMA, 64, 64, 64, 4, 16, 2, 2, 2, 0.27, false},
        {dtg::KF_DMA, 192, 256, 64, 2, 16, 2, 4, 1, 0.85, true},
    };
    const bool row_major_vec = kernel_layout(p) == 0 && vec_shape_ok(p);
    const C* best = nullptr;
    double best_t = 0.0;
    for (const C& c : ladder) {
        if (c.row_major_only && !row_major_vec) continue;
        const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
        const double t = static_cast<double>(cdiv(tiles, static_cast<int64_t>(dev.cu_count) * c.per_cu)) * c.cost;
        if (!best || t < best_t) {
            best = &c;
            best_t = t;
        }
    }
    // K slices of the 4-stage 128 x 128 tile (one workgroup per CU) when at
    // least two slices of >= 16 K steps fit in the CUs and the estimate says
    // they win: few tiles with a deep K, and the wide, short problems
    // (M <= 256) the ladder serves poorly.  Slices of at least 16 K steps,
    // at most 16 (the last arriver reads them all).  Estimate, in K steps of
    // a full round of 256 x 256 tiles: the ladder's best takes best_t x nkt,
    // the slices 0.43 x nkt / S plus ~3.3 for the fused reduce (a few
    // dependent memory round trips, ~5 us): 768^2 x 2048 stays on 64 x 64
    // tiles (12.1 us; 2 slices 16.4 us), 768^2 x 8192 takes 7 slices (24.9
    // us; 64 x 64 34.3 us).  Measured (bf16, medians): 512^2 x 32768 36.5 us with 16 slices
    // (2-stage tile 42.0, unsplit 322), 1024^2 x 16384 42.6 us with 4 (64 x 64
    // 65.0), 768^2 x 8192 23.9 us with 4 (64 x 64 34.3), 192 x 8192 x 8192
    // 38.1 us with 2 (64 x 64 46.6), 256 x 8192 x 8192 48.4 us with 2
    // (64 x 64 80.3), 64 x 8192 x 8192 34.7 us with 4, 128 x 4096 x 4096
    // 16.8 us with 4 (64 x 64 19.1); 1024^2 x 4096 20.7 us with 4 (64 x 64
    // 20.0).
    const C& split = ladder[3];
    const int64_t tiles = cdiv(M, split.bm) * cdiv(N, split.bn);
    const int64_t nkt = cdiv(K, split.bk);
    if (allow_ws && tiles <= dtg::kMaxCounters && p->dtype != GEMM_I8) {   // int8: no K slices
        int64_t s = dev.cu_count / tiles;
        if (s > nkt / 16) s = nkt / 16;
        if (s > 16) s = 16;
        const double steps = static_cast<double>(nkt);
        if (s > 1 && split.cost * steps / static_cast<double>(s) + 3.3 < best_t * steps) {
            // When K allows the 128 x 128 tiles only a few slices (<= 4) and
            // the 4-wave 64 x 64 tiles can still take two or more, the
            // smaller tile's slices win: swept (bf16, every compiled
            // variant, interleaved races) 64 x 4096^2 11.1 us with 4 of them
            // (128 x 128 with 4 slices 16.1), 64 x 8192^2 25.1 us with 2
            // (30.3), 128 x 4096^2 13.9 us with 2 (16.5); with many slices
            // the larger tile stays (512^2 x 32768: 128 x 128 with 16 slices
            // 35.1 us, 64 x 64 with 4 41.3).
            const C& small = ladder[5];
            const int64_t tiles64 = cdiv(M, small.bm) * cdiv(N, small.bn);
            int64_t s64 = dev.cu_count / tiles64;
            if (s64 > nkt / 16) s64 = nkt / 16;
            if (s64 > 16) s64 = 16;
            if (s <= 4 && s64 > 1 && tiles64 <= dtg::kMaxCounters) {
                gemm_config c = cfg_of(small.fam, small.bm, small.bn, small.bk, small.st, small.mf, small.wm, small.wn);
                c.splitk = static_cast<int32_t>(s64);
                return c;
            }
            gemm_config c = cfg_of(split.fam, split.bm, split.bn, split.bk, split.st, split.mf, split.wm, split.wn);
            c.splitk = static_cast<int32_t>(s);
            return c;
        }
    }
    // Stream-K (kernel 6) is not planned: measured against these tiles it
    // loses at every shape tried (3072^2 x 4096 113.6 us against 68.6 for
    // 192 x 256, 5120^2 x 4096 261 against 172 for 256 x 256): each cut tile
    // moves 256 KiB fp32 parts through memory, and ranges at staggered K
    // offsets lose the L2 reuse of A and B panels that tiles in lockstep get.
    return cfg_of(best->fam, best->bm, best->bn, best->bk, best->st, best->mf, best->wm, best->wn);
}

gemm_status plan_impl(const gemm_problem* given, const gemm_device_info* dev, const gemm_config* force,
                      gemm_plan** out, bool allow_ws = true) {
    if (!out) return fail(GEMM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    gemm_status st = validate(given);
    if (st != GEMM_OK) return st;
    gemm_problem view;
    st = kernel_view(given, &view);
    if (st != GEMM_OK) return st;
    const gemm_problem* prob = &view;   // everything below plans in the kernels' units
    if (!dev) return fail(GEMM_ERR_INVALID_ARG, "device info is NULL");
    if (dev->cu_count <= 0 || dev->lds_per_wg <= 0)
        return fail(GEMM_ERR_INVALID_ARG, "device info has no CUs or no LDS");

    const bool vec = vec_shape_ok(prob);
    int group_m = 8, xcd = 1;
    gemm_config want;
    bool tuned = false;
    if (vec && layout_of(prob) == 0) {
        for (const TunedKey& t : tuned_table()) {
            if (t.M == prob->M && t.N == prob->N && t.K == prob->K && t.dtype == prob->dtype &&
                t.has_c == prob->has_c && (allow_ws || t.cfg.splitk <= 1) &&
                find_entry(t.cfg, prob->dtype, 1, *dev, prob)) {
                want = t.cfg;
                group_m = t.group_m;
                xcd = t.xcd;
                tuned = true;
                break;
            }
        }
    }
    if (!tuned) want = heuristic(prob, *dev, &group_m, allow_ws);
    if (force) {
        // Any forced tile field replaces the planner's tile; the tile fields
        // left at 0 are then free (the first compiled variant that matches).
        const gemm_config& f = *force;
        if (f.group_m < 0 || f.xcd_remap < 0 || f.xcd_remap > 2)
            return fail(GEMM_ERR_INVALID_ARG, "group_m must be >= 0 and xcd_remap one of 0, 1, 2");
        if (f.bm || f.bn || f.bk || f.mfma || f.waves_m || f.waves_n || f.stages || f.kernel || f.splitk)
            want = f;
        if (f.group_m) group_m = f.group_m;
        if (f.xcd_remap) xcd = (f.xcd_remap == GEMM_XCD_ON);
    }
    const dtg::KernelEntry* e = nullptr;
    if (vec) e = find_entry(want, prob->dtype, 1, *dev, prob);
    if (!e && vec && !tuned && (!force || force->kernel == 0) && want.kernel == dtg::KF_DMA) {
        // no direct-to-LDS variant fits (offset range, row strides): the
        // register-staged kernel with the same tile, any wave grid and depth
        gemm_config w2 = cfg_of(dtg::KF_TILE, want.bm, want.bn, 0, 0, want.mfma, 0, 0);
        e = find_entry(w2, prob->dtype, 1, *dev, prob);
    }
    const dtg::KernelEntry* fb =
        find_entry(cfg_of(dtg::KF_TILE, 0, 0, 0, 0, 16, 0, 0), prob->dtype, 0, *dev, prob);
    const bool unforced = !force || (!force->kernel && !force->bm && !force->bn && !force->bk && !force->mfma &&
                                     !force->waves_m && !force->waves_n && !force->stages && !force->splitk);
    if (!e && vec && unforced && !tuned) {
        // no vector variant for this layout, tile or stride: the element-wise path
        e = fb;
    }
    if (!e) {
        if (!vec && (!force || want.kernel == 0 || want.kernel == dtg::KF_TILE)) {
            // element-wise path: any shape, any alignment (16x16x32 instruction)
            if (force && (want.bm || want.bn || want.bk || want.mfma == 32))
                e = find_entry(want, prob->dtype, 0, *dev, prob);
            else
                e = fb;
        }
        if (!e)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "no compiled kernel for bm=%d bn=%d bk=%d stages=%d mfma=%d waves=%dx%d kernel=%d "
                        "(dtype %d, vector path %d) within %lld bytes of LDS",
                        want.bm, want.bn, want.bk, want.stages, want.mfma, want.waves_m, want.waves_n,
                        want.kernel, (int)prob->dtype, (int)vec, (long long)dev->lds_per_wg);
    }
    // one row of tiles: the streamed-B twin where one is compiled
    if (e->family == dtg::KF_DMA && cdiv(prob->M, e->bm) == 1) e = stream_b_twin(e, *dev, prob);
    if (e->family == dtg::KF_SKINNY && prob->M > e->bm)
        return fail(GEMM_ERR_UNSUPPORTED, "this skinny kernel runs M <= %d only (M=%lld)", e->bm,
                    (long long)prob->M);
    int splits = 1;
    int64_t sk_groups = 0;   // stream-K: workgroups the (tile, K step) iterations are dealt to
    if (e->family == dtg::KF_DMA_SK) {
        if (!allow_ws) return fail(GEMM_ERR_UNSUPPORTED, "stream-K needs a workspace");
        const int64_t total = cdiv(prob->M, e->bm) * cdiv(prob->N, e->bn) * cdiv(prob->K, e->bk);
        sk_groups = want.splitk >= 1 ? want.splitk : dev->cu_count;
        if (want.splitk < 1 && sk_groups > total / 16) sk_groups = total / 16;
        if (sk_groups < 1) sk_groups = 1;
        // 2 W fp32 tiles of parts, addressed with 32-bit offsets from one descriptor
        const int64_t part_bytes = 2 * sk_groups * static_cast<int64_t>(e->bm) * e->bn * 4;
        if (sk_groups > total || sk_groups > dtg::kMaxCounters || total * sk_groups >= (int64_t(1) << 31) ||
            part_bytes >= (int64_t(1) << 31) - 4096)
            return fail(GEMM_ERR_UNSUPPORTED,
                        "stream-K takes 1 to min(%d, tiles x K steps = %lld) workgroups, with tiles x K steps x "
                        "workgroups and the parts' bytes below 2^31 (splitk=%d)",
                        dtg::kMaxCounters, (long long)total, want.splitk);
    }
    if (e->family == dtg::KF_SKINNY || e->family == dtg::KF_DMA) {
        splits = want.splitk > 0 ? want.splitk : 1;
        if (splits > 64) return fail(GEMM_ERR_UNSUPPORTED, "at most 64 K slices (splitk=%d)", splits);
        if (e->splitk > 0 && splits > e->splitk)
            return fail(GEMM_ERR_UNSUPPORTED, "%s takes at most %d K slices (splitk=%d)", e->name, e->splitk,
                        splits);
        if (splits > 1 && !allow_ws)
            return fail(GEMM_ERR_UNSUPPORTED, "K slices across workgroups need a workspace");
    }
    gemm_plan* pl = new (std::nothrow) gemm_plan;
    if (!pl) return fail(GEMM_ERR_INVALID_ARG, "out of host memory");
    pl->prob = *given;
    pl->view = view;
    pl->dev = *dev;
    pl->entry = e;
    pl->fallback = fb;
    pl->num_pid_m = cdiv(prob->M, e->bm);
    pl->num_pid_n = cdiv(prob->N, e->bn);
    pl->grid = e->family == dtg::KF_DMA_SK ? sk_groups : pl->num_pid_m * pl->num_pid_n * splits;
    pl->ws_bytes = e->family == dtg::KF_SKINNY ? dtg::skinny_workspace_bytes(pl->num_pid_n, e->bm, e->bn, splits)
                   : e->family == dtg::KF_DMA
                       ? dtg::dma_workspace_bytes(pl->num_pid_m * pl->num_pid_n, e->bm, e->bn, splits)
                   : e->family == dtg::KF_DMA_SK
                       ? dtg::dma_sk_workspace_bytes(pl->num_pid_m * pl->num_pid_n, e->bm, e->bn, sk_groups)
                       : 0;
    if (pl->ws_bytes < 0) {
        delete pl;
        return fail(GEMM_ERR_UNSUPPORTED, "K slices across workgroups support at most %d column slabs or tiles",
                    dtg::kMaxCounters);
    }
    // a band taller than the grid orders the tiles exactly as a band of the
    // whole grid: clamping keeps the kernels' band arithmetic in 32 bits
    if (group_m < 1) group_m = 1;
    if (group_m > pl->num_pid_m) group_m = static_cast<int>(pl->num_pid_m);
    gemm_config& c = pl->cfg;
    c = cfg_of(e->family, e->bm, e->bn, e->bk, e->stages, e->mfma, e->waves_m, e->waves_n);
    c.splitk = e->family == dtg::KF_DMA_SK ? static_cast<int32_t>(sk_groups) : splits;
    c.group_m = group_m;
    c.xcd_remap = (xcd && dev->xcd_count > 1) ? GEMM_XCD_ON : GEMM_XCD_OFF;
    if (log_enabled()) {
        char buf[512];
        gemm_plan_describe(pl, buf, sizeof buf);
        fprintf(stderr, "[gemm] M=%lld N=%lld K=%lld dtype=%d has_c=%d: %s%s\n", (long long)given->M,
                (long long)given->N, (long long)given->K, (int)given->dtype, (int)given->has_c, buf,
                tuned ? " (tuned)" : "");
    }
    *out = pl;
    return ok();
}

std::mutex g_dev_mu;
std::map<int, gemm_device_info> g_dev_cache;

gemm_status device_info_cached(int device, gemm_device_info* info) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_dev_cache.find(device);
    if (it != g_dev_cache.end()) {
        *info = it->second;
        return ok();
    }
    gemm_status st = gemm_device_query(device, info);
    if (st == GEMM_OK) g_dev_cache[device] = *info;
    return st;
}

// byte range [lo, hi) of a rows x cols matrix of elem-byte elements with
// strides (rs, cs) in elements
void span(const void* p, int64_t rows, int64_t cols, int64_t rs, int64_t cs, int64_t elem, uintptr_t* lo,
          uintptr_t* hi) {
    *lo = reinterpret_cast<uintptr_t>(p);
    *hi = *lo + static_cast<uintptr_t>(((rows - 1) * rs + (cols - 1) * cs + 1) * elem);
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

struct CacheKey {
    int device;
    int64_t f[12];
    bool operator<(const CacheKey& o) const {
        if (device != o.device) return device < o.device;
        return memcmp(f, o.f, sizeof f) < 0;
    }
};
std::mutex g_cache_mu;
std::map<CacheKey, std::unique_ptr<gemm_plan>> g_cache;

}  // namespace

namespace dtg {
gemm_status record_error(gemm_status st, const char* msg) {
    g_err = msg;
    return st;
}
gemm_status cached_device_info(int device, gemm_device_info* info) { return device_info_cached(device, info); }
}  // namespace dtg

extern "C" {

const char* gemm_status_string(gemm_status s) {
    switch (s) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
        case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
        case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE";
    }
    return "GEMM_ERR_UNKNOWN";
}

const char* gemm_last_error(void) { return g_err.c_str(); }

gemm_status gemm_device_query(int device, gemm_device_info* info) {
    if (!info) return fail(GEMM_ERR_INVALID_ARG, "info is NULL");
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return fail(GEMM_ERR_HIP, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
    memset(info, 0, sizeof *info);
    int arch = 0;
    if (sscanf(prop.gcnArchName, "gfx%d", &arch) != 1) arch = 0;
    info->arch = arch;
    info->cu_count = prop.multiProcessorCount;
    info->clock_khz = prop.clockRate;
    info->lds_per_cu = static_cast<int64_t>(prop.maxSharedMemoryPerMultiProcessor);
    info->lds_per_wg = static_cast<int64_t>(prop.sharedMemPerBlock);
    if (prop.sharedMemPerBlockOptin > prop.sharedMemPerBlock)
        info->lds_per_wg = static_cast<int64_t>(prop.sharedMemPerBlockOptin);
    if (info->lds_per_cu > 0 && info->lds_per_wg > info->lds_per_cu) info->lds_per_wg = info->lds_per_cu;
    info->wave_size = prop.warpSize;
    int xccs = 1;
    if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || xccs < 1)
        xccs = 1;
    info->xcd_count = xccs;
    if (arch != 950)
        return fail(GEMM_ERR_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950", device,
                    prop.gcnArchName);
    if (prop.warpSize != 64) return fail(GEMM_ERR_UNSUPPORTED, "wave size %d, expected 64", prop.warpSize);
    return ok();
}

gemm_status gemm_plan_create_for(const gemm_problem* prob, const gemm_device_info* info,
                                 const gemm_config* force, gemm_plan** out) {
    return plan_impl(prob, info, force, out);
}

gemm_status gemm_plan_create(const gemm_problem* prob, int device, const gemm_config* force,
                             gemm_plan** out) {
    if (out) *out = nullptr;
    gemm_status st = validate(prob);
    if (st != GEMM_OK) return st;
    gemm_device_info info;
    st = device_info_cached(device, &info);
    if (st != GEMM_OK) return st;
    return plan_impl(prob, &info, force, out);
}

void gemm_plan_destroy(gemm_plan* plan) { delete plan; }

gemm_status gemm_plan_config(const gemm_plan* plan, gemm_config* out) {
    if (!plan || !out) return fail(GEMM_ERR_INVALID_ARG, "plan or out is NULL");
    *out = plan->cfg;
    return ok();
}

gemm_status gemm_plan_launch(const gemm_plan* plan, int64_t* grid, int32_t* threads, int64_t* lds) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    if (grid) *grid = plan->grid;
    if (threads) *threads = plan->entry->threads;
    if (lds) *lds = plan->entry->lds_bytes;
    return ok();
}

gemm_status gemm_plan_describe(const gemm_plan* plan, char* buf, size_t len) {
    if (!plan || !buf || len == 0) return fail(GEMM_ERR_INVALID_ARG, "plan or buf is NULL");
    const gemm_config& c = plan->cfg;
    snprintf(buf, len,
             "kernel=%s bm=%d bn=%d bk=%d stages=%d mfma=%d waves=%dx%d group_m=%d splitk=%d xcd_remap=%d "
             "grid=%lld threads=%d lds=%lld vec=%d layout=%d",
             plan->entry->name, c.bm, c.bn, c.bk, c.stages, c.mfma, c.waves_m, c.waves_n, c.group_m,
             c.splitk, c.xcd_remap, (long long)plan->grid, plan->entry->threads,
             (long long)plan->entry->lds_bytes, plan->entry->vec, kernel_layout(&plan->view));
    return ok();
}

gemm_status gemm_workspace_size(const gemm_plan* plan, size_t* bytes) {
    if (!plan || !bytes) return fail(GEMM_ERR_INVALID_ARG, "plan or bytes is NULL");
    *bytes = static_cast<size_t>(plan->ws_bytes);
    return ok();
}

gemm_status gemm_workspace_init(const gemm_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    if (plan->ws_bytes == 0) return ok();
    if (!workspace || workspace_bytes < static_cast<size_t>(plan->ws_bytes))
        return fail(GEMM_ERR_WORKSPACE, "workspace of %zu bytes given, %lld needed", workspace_bytes,
                    (long long)plan->ws_bytes);
    hipError_t e = dtg::zero_words(workspace, plan->ws_bytes / 4, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "workspace zero fill: %s", hipGetErrorString(e));
    return ok();
}

gemm_status gemm_run(const gemm_plan* plan, const void* A, const void* B, const void* C, void* D,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    const gemm_problem& p = plan->prob;
    if (p.has_c && !C) return fail(GEMM_ERR_INVALID_ARG, "problem has C but C is NULL");
    if (!p.has_c && C) return fail(GEMM_ERR_INVALID_ARG, "C given but the problem has has_c = 0");
    if (p.M == 0 || p.N == 0) return ok();
    if (!D) return fail(GEMM_ERR_INVALID_ARG, "D is NULL");
    if (p.K > 0 && (!A || !B)) return fail(GEMM_ERR_INVALID_ARG, "A or B is NULL");
    const bool i8 = p.dtype == GEMM_I8;
    const int64_t eab = i8 ? 1 : 2, ecd = i8 ? 4 : 2;   // element bytes of A, B and of C, D
    uintptr_t d0, d1;
    span(D, p.M, p.N, p.sd_m, p.sd_n, ecd, &d0, &d1);
    if (p.K > 0) {
        uintptr_t a0, a1, b0, b1;
        span(A, p.M, p.K, p.sa_m, p.sa_k, eab, &a0, &a1);
        span(B, p.K, p.N, p.sb_k, p.sb_n, eab, &b0, &b1);
        if (overlaps(d0, d1, a0, a1)) return fail(GEMM_ERR_INVALID_ARG, "D overlaps A");
        if (overlaps(d0, d1, b0, b1)) return fail(GEMM_ERR_INVALID_ARG, "D overlaps B");
    }
    if (p.has_c) {
        uintptr_t c0, c1;
        span(C, p.M, p.N, p.sc_m, p.sc_n, ecd, &c0, &c1);
        const bool same = (C == D) && (p.sc_m == p.sd_m || p.M == 1);
        if (!same && overlaps(d0, d1, c0, c1))
            return fail(GEMM_ERR_INVALID_ARG, "D overlaps C (only D == C with equal strides is allowed)");
    }
    const dtg::KernelEntry* e = plan->entry;
    const bool needs_ws = plan->ws_bytes > 0;
    if (needs_ws && (!workspace || workspace_bytes < static_cast<size_t>(plan->ws_bytes)))
        return fail(GEMM_ERR_WORKSPACE, "plan needs a workspace of %lld bytes (%zu given)",
                    (long long)plan->ws_bytes, workspace ? workspace_bytes : static_cast<size_t>(0));
    if (needs_ws && (reinterpret_cast<uintptr_t>(workspace) & 255))
        return fail(GEMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (e->vec && p.K > 0 &&
        ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(B) & 15))) {
        if (!plan->fallback)
            return fail(GEMM_ERR_UNSUPPORTED, "int8 operands must be 16-byte aligned (no element-wise int8 path)");
        e = plan->fallback;   // element-wise loads; bitwise identical for 16x16x32 plans
    }
    const gemm_problem& v = plan->view;   // A, B and K in the kernels' units
    dtg::KArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = static_cast<const uint16_t*>(C);
    a.D = static_cast<uint16_t*>(D);
    a.M = static_cast<int32_t>(p.M);
    a.N = static_cast<int32_t>(p.N);
    a.K = static_cast<int32_t>(v.K);
    a.num_pid_m = static_cast<int32_t>((p.M + e->bm - 1) / e->bm);
    a.num_pid_n = static_cast<int32_t>((p.N + e->bn - 1) / e->bn);
    a.group_m = plan->cfg.group_m;
    a.xcds = (plan->cfg.xcd_remap == GEMM_XCD_ON) ? plan->dev.xcd_count : 1;
    a.has_c = p.has_c;
    a.lda = v.sa_m;
    a.ldb = v.sb_k;
    a.ldc = p.has_c ? p.sc_m : 0;
    a.ldd = p.sd_m;
    a.sak = v.sa_k;
    a.sbn = v.sb_n;
    a.splits = (e == plan->entry && (e->family == dtg::KF_SKINNY || e->family == dtg::KF_DMA))
                   ? plan->cfg.splitk
                   : 1;   // the element-wise fallback runs the whole K range per tile
    a.ws = workspace;
    const int64_t grid = e == plan->entry ? plan->grid : static_cast<int64_t>(a.num_pid_m) * a.num_pid_n;
    hipError_t err = e->launch(a, grid, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(GEMM_ERR_HIP, "launch of %s: %s", e->name, hipGetErrorString(err));
    return ok();
}

gemm_status gemm(const void* A, const void* B, const void* C, void* D, int64_t M, int64_t N, int64_t K,
                 const int64_t strides[8], gemm_dtype dtype, int32_t has_c, void* stream) {
    if (!strides) return fail(GEMM_ERR_INVALID_ARG, "strides is NULL");
    gemm_problem p;
    p.M = M; p.N = N; p.K = K;
    p.sa_m = strides[0]; p.sa_k = strides[1]; p.sb_k = strides[2]; p.sb_n = strides[3];
    p.sc_m = strides[4]; p.sc_n = strides[5]; p.sd_m = strides[6]; p.sd_n = strides[7];
    p.dtype = dtype;
    p.has_c = has_c;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    CacheKey key;
    key.device = device;
    const int64_t f[12] = {M, N, K, p.sa_m, p.sa_k, p.sb_k, p.sb_n,
                           has_c ? p.sc_m : 0, has_c ? p.sc_n : 0, p.sd_m, p.sd_n,
                           (int64_t)dtype * 2 + has_c};
    memcpy(key.f, f, sizeof f);
    const gemm_plan* plan = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = g_cache.find(key);
        if (it != g_cache.end()) {
            plan = it->second.get();
        } else {
            gemm_plan* np = nullptr;
            gemm_device_info info;
            gemm_status st = device_info_cached(device, &info);
            if (st != GEMM_OK) return st;
            st = plan_impl(&p, &info, nullptr, &np, /*allow_ws=*/false);
            if (st != GEMM_OK) return st;
            g_cache[key].reset(np);
            plan = np;
        }
    }
    return gemm_run(plan, A, B, C, D, nullptr, 0, stream);
}

void gemm_cache_clear(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache.clear();
}

int64_t gemm_lds_bytes(int32_t bm, int32_t bn, int32_t bk, int32_t stages, gemm_dtype dtype) {
    if (bm <= 0 || bn <= 0 || bk <= 0 || stages <= 0) return -1;
    if (dtype != GEMM_F16 && dtype != GEMM_BF16 && dtype != GEMM_I8) return -1;
    return static_cast<int64_t>(stages) * (bm + bn) * bk * (dtype == GEMM_I8 ? 1 : 2);
}

gemm_status gemm_tile_of_workgroup(int64_t wg, int64_t num_pid_m, int64_t num_pid_n, int32_t group_m,
                                   int32_t xcd_count, int64_t* pid_m, int64_t* pid_n) {
    if (!pid_m || !pid_n) return fail(GEMM_ERR_INVALID_ARG, "output pointer is NULL");
    if (num_pid_m <= 0 || num_pid_n <= 0 || group_m <= 0 || xcd_count <= 0)
        return fail(GEMM_ERR_INVALID_ARG, "grid sizes, group_m and xcd_count must be positive");
    if (wg < 0 || wg >= num_pid_m * num_pid_n) return fail(GEMM_ERR_INVALID_ARG, "workgroup outside the grid");
    const int64_t gm = group_m < num_pid_m ? group_m : num_pid_m;   // as the planners clamp it
    dtg::tile_of_workgroup<int64_t>(wg, num_pid_m, num_pid_n, gm, xcd_count, pid_m, pid_n);
    return ok();
}

gemm_status gemm_streamk_pieces(int32_t tiles, int32_t k_steps, int32_t workgroups, int32_t wg, int32_t* out,
                                int32_t max_pieces, int32_t* count) {
    if (!count || (max_pieces > 0 && !out)) return fail(GEMM_ERR_INVALID_ARG, "output pointer is NULL");
    const int64_t total = static_cast<int64_t>(tiles) * k_steps;
    if (tiles <= 0 || k_steps <= 0 || workgroups <= 0 || wg < 0 || wg >= workgroups || workgroups > total ||
        total * workgroups >= (int64_t(1) << 31))
        return fail(GEMM_ERR_INVALID_ARG, "need 0 <= wg < workgroups <= tiles x k_steps < 2^31 / workgroups");
    const uint32_t T = static_cast<uint32_t>(total), W = static_cast<uint32_t>(workgroups);
    uint32_t it = dtg::sk_range_start(static_cast<uint32_t>(wg), T, W);
    const uint32_t end = dtg::sk_range_start(static_cast<uint32_t>(wg) + 1, T, W);
    int32_t n = 0;
    while (it < end) {
        const dtg::SkPiece q = dtg::sk_piece(it, end, T, static_cast<uint32_t>(k_steps), W);
        if (n < max_pieces) {
            int32_t* o = out + 6 * n;
            o[0] = static_cast<int32_t>(q.tile);
            o[1] = static_cast<int32_t>(q.kt0);
            o[2] = static_cast<int32_t>(q.kt1);
            o[3] = static_cast<int32_t>(q.part);
            o[4] = static_cast<int32_t>(q.nparts);
            o[5] = q.nparts == 1 ? -1 : static_cast<int32_t>(q.part == 0 ? q.slot0 : q.slot1 + q.part);
        }
        ++n;
        it = q.next;
    }
    *count = n;
    return ok();
}

}  // extern "C"
