// C ABI of the block-scaled (MX) GEMM: validation, tile choice and launch.
// Declarations and the contract of every entry point are in include/gemm_mx.h.
//
// The tile choice follows the 16-bit planner: the largest 8-wave tile that
// still gives at least half of the CUs a workgroup, else 128 x 128 ("Tuning
// Triton kernels", sections 3-4: the choice is keyed on every tiled dimension
// and separates regimes).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include "../../include/gemm_mx.h"
#include "api_internal.h"
#include "kernels.h"
#include "kernels_mx.h"

struct gemm_mx_plan {
    gemm_mx_problem prob;
    gemm_device_info dev;
    gemm_config cfg;
    const dtg::MxEntry* entry;
    int64_t num_pid_m, num_pid_n, grid;
    int64_t ws_bytes;
};

namespace {

gemm_status fail(gemm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gemm_status fail(gemm_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return dtg::record_error(st, buf);
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
bool fmt_ok(int f) {
    return f == GEMM_MX_E4M3 || f == GEMM_MX_E5M2 || f == GEMM_MX_E2M3 || f == GEMM_MX_E3M2 || f == GEMM_MX_E2M1;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int elem_bits(int f) { return f == GEMM_MX_E2M1 ? 4 : (f == GEMM_MX_E2M3 || f == GEMM_MX_E3M2) ? 6 : 8; }

// Bytes of k of one row of a format: K elements of 8, 6 or 4 bits.
int64_t row_bytes(int64_t K, int fmt) { return K * elem_bits(fmt) / 8; }

// Pairs of one width (8-bit with 8-bit, E2M1 with E2M1) have the tile
// kernel's full variant table; the others (an FP6 operand, or 8-bit with
// 4-bit) its 256 x 256, 128 x 128, 64 x 64 and 32 x 64 variants.
bool one_width_pair(const gemm_mx_problem* p) {
    const int a = elem_bits(p->fmt_a), b = elem_bits(p->fmt_b);
    return a == b && a != 6;
}

gemm_status validate(const gemm_mx_problem* p) {
    if (!p) return fail(GEMM_ERR_INVALID_ARG, "problem is NULL");
    if (p->M < 0 || p->N < 0 || p->K < 0)
        return fail(GEMM_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld", (long long)p->M, (long long)p->N,
                    (long long)p->K);
    if (!fmt_ok(p->fmt_a) || !fmt_ok(p->fmt_b))
        return fail(GEMM_ERR_INVALID_ARG,
                    "element formats %d / %d: expected GEMM_MX_E4M3, _E5M2, _E2M3, _E3M2 or _E2M1", (int)p->fmt_a,
                    (int)p->fmt_b);
    if (p->out != GEMM_MX_OUT_F16 && p->out != GEMM_MX_OUT_BF16 && p->out != GEMM_MX_OUT_F32)
        return fail(GEMM_ERR_INVALID_ARG, "output type %d is not a gemm_mx_out value", (int)p->out);
    if (p->has_c != 0 && p->has_c != 1)
        return fail(GEMM_ERR_INVALID_ARG, "has_c must be 0 or 1, got %d", (int)p->has_c);
    if (p->M > kMaxDim || p->N > kMaxDim || p->K > kMaxDim)
        return fail(GEMM_ERR_UNSUPPORTED, "dimensions above 2^31-1 are not supported");
    // K granularity: a whole 16-byte chunk of 8-bit elements (16 k), a whole
    // 32-k block of 6- and 4-bit ones (24 and 16 bytes)
    const int64_t kq = (elem_bits(p->fmt_a) == 8 && elem_bits(p->fmt_b) == 8) ? 16 : 32;
    if (p->K % kq != 0)
        return fail(GEMM_ERR_UNSUPPORTED, "K=%lld must be a multiple of %lld for these element formats",
                    (long long)p->K, (long long)kq);
    const int64_t kba = row_bytes(p->K, p->fmt_a), kbb = row_bytes(p->K, p->fmt_b), nblk = cdiv(p->K, 32);
    const int64_t kb = kba > kbb ? kba : kbb;
    if (p->lda < 0 || p->ldb < 0 || p->ldsa < 0 || p->ldsb < 0 || p->ldc < 0 || p->ldd < 0)
        return fail(GEMM_ERR_INVALID_ARG, "negative stride");
    if (p->lda % 16 || p->ldb % 16)
        return fail(GEMM_ERR_UNSUPPORTED, "lda=%lld and ldb=%lld must be multiples of 16 bytes", (long long)p->lda,
                    (long long)p->ldb);
    if (p->ldsa % 4 || p->ldsb % 4)
        return fail(GEMM_ERR_UNSUPPORTED, "ldsa=%lld and ldsb=%lld must be multiples of 4 bytes",
                    (long long)p->ldsa, (long long)p->ldsb);
    if ((p->M > 1 && p->lda < kba) || (p->N > 1 && p->ldb < kbb))
        return fail(GEMM_ERR_INVALID_ARG, "lda / ldb below the %lld / %lld bytes of a row", (long long)kba,
                    (long long)kbb);
    if ((p->M > 0 && p->ldsa < nblk) || (p->N > 0 && p->ldsb < nblk))
        return fail(GEMM_ERR_INVALID_ARG, "ldsa / ldsb below ceil(K/32) = %lld", (long long)nblk);
    if (p->M > 1 && p->N > 0 && p->ldd < p->N)
        return fail(GEMM_ERR_INVALID_ARG, "D row stride %lld < N=%lld makes output rows overlap",
                    (long long)p->ldd, (long long)p->N);
    // 32-bit buffer offsets and ranges cover one tile's rows of every operand
    // plus the K extent (descriptors move along k from the tile's corner)
    const int64_t lim = (int64_t(1) << 31) - 4096;
    if (256 * p->lda + kb >= lim || 256 * p->ldb + kb >= lim || 256 * p->ldsa + nblk >= lim ||
        256 * p->ldsb + nblk >= lim)
        return fail(GEMM_ERR_UNSUPPORTED, "row strides too large for 32-bit tile offsets");
    return GEMM_OK;
}

const dtg::MxEntry* find_entry(const gemm_config& w, const gemm_mx_problem* p, const gemm_device_info& dev) {
    int n = 0, np = 0, nd = 0;
    const dtg::MxEntry* t = dtg::mx_kernel_table(&n);
    const dtg::MxEntry* tp = dtg::mx_pair_kernel_table(&np);
    const dtg::MxEntry* td = dtg::mx_direct_kernel_table(&nd);
    for (int i = 0; i < n + np + nd; ++i) {
        const dtg::MxEntry* e = i < n ? &t[i] : i < n + np ? &tp[i - n] : &td[i - n - np];
        if (e->fmt_a != p->fmt_a || e->fmt_b != p->fmt_b || e->lds_bytes > dev.lds_per_wg) continue;
        if (w.kernel && w.kernel != e->kind) continue;
        if ((w.bm && w.bm != e->bm) || (w.bn && w.bn != e->bn) || (w.stages && w.stages != e->stages) ||
            (w.waves_m && w.waves_m != e->waves_m) || (w.waves_n && w.waves_n != e->waves_n) ||
            (w.bk && w.bk != e->bk) || (w.mfma && w.mfma != e->mfma) || (w.splitk > e->splitk))
            continue;
        return e;
    }
    return nullptr;
}

gemm_status plan_impl(const gemm_mx_problem* prob, const gemm_device_info* dev, const gemm_config* force,
                      gemm_mx_plan** out) {
    if (!out) return fail(GEMM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    gemm_status st = validate(prob);
    if (st != GEMM_OK) return st;
    if (!dev || dev->cu_count <= 0 || dev->lds_per_wg <= 0)
        return fail(GEMM_ERR_INVALID_ARG, "device info missing, or without CUs or LDS");
    gemm_config want;
    memset(&want, 0, sizeof want);
    int group_m = 8, xcd = 1;
    // k per K step of the tile kernel
    const int64_t bke = (prob->fmt_a == GEMM_MX_E2M1 && prob->fmt_b == GEMM_MX_E2M1) ? 256 : 128;
    const int64_t nkt = cdiv(prob->K, bke);
    // K slices: enough workgroups for the CUs, at least 2 K steps per slice, at most 16
    auto slices = [&](int64_t tiles, int64_t min_steps) {
        int64_t s = dev->cu_count / (tiles > 0 ? tiles : 1);
        if (s > nkt / min_steps) s = nkt / min_steps;
        if (s > 16) s = 16;
        if (tiles > dtg::kMaxCounters) s = 1;
        return static_cast<int32_t>(s > 1 ? s : 1);
    };
    if (prob->M <= 32) {
        // decode regime: 32-row slabs of 64 columns, K sliced to fill the CUs
        // (more slices per tile cost more in the fp32 partial-tile reduction
        // than they gain in load parallelism)
        want.bm = 32;
        want.bn = 64;
        want.splitk = slices(cdiv(prob->N, 64), 2);
    } else {
        // Tile by estimated time: ceil(tiles / CUs) rounds of workgroups times
        // the tile's cost per round relative to 256 x 256, fitted to forced
        // runs (E4M3 / E2M1 medians): 4096^3 and 3072^2 x 4096 pick 256 x 256
        // (69 / 54 us; 256 x 128 90 / 75 us), 4096 x 2048 x 8192 256 x 128 or
        // 128 x 256 (79 us; 256 x 256 99 us), 2560^2 x 4096 128 x 256 (40 us;
        // 128 x 128 48 us, 256 x 256 52 us), 2048^2 x 4096 128 x 128 (27 us;
        // 256 x 128 37 us, 256 x 256 50 us), 1024^2 x 4096 64 x 64 (12.6 us;
        // 128 x 128 22.8 us), 768^2 x 4096 64 x 64 (12.1 us; 20.3 us); 192 x 256
        // where 256 x 256 leaves CUs idle and the mid tiles need a second
        // round: 3072^2 x 4096 49.3 / 31.6 us (256 x 256 54.9 / 34.4),
        // 4000 x 3000 x 1024 21.5 / 17.6 us (23.6 / 18.8), bitwise the same.
        struct T { int bm, bn; double cost; };
        static const T ladder[] = {{256, 256, 1.0}, {256, 128, 0.65}, {128, 256, 0.65}, {128, 128, 0.4},
                                   {64, 64, 0.25},   {192, 256, 0.9}};
        const T* best = nullptr;
        double best_t = 0.0;
        const bool full = one_width_pair(prob);
        for (const T& t : ladder) {
            // pairs outside the one-width table have the square tiles only
            if (!full && t.bm != t.bn) continue;
            const int64_t tiles = cdiv(prob->M, t.bm) * cdiv(prob->N, t.bn);
            const double est = static_cast<double>(cdiv(tiles, dev->cu_count)) * t.cost;
            if (!best || est < best_t) {
                best = &t;
                best_t = est;
            }
        }
        want.bm = best->bm;
        want.bn = best->bn;
        // K slices of 128 x 128 tiles when even 64 x 64 tiles leave more than
        // half of the CUs idle and K gives at least 4 slices of 8 K steps
        // (E4M3 512^2 x 16384: 27.5 us with 16 slices, 41.0 us as 64 x 64;
        // 1024^2 x 4096: 64 x 64 12.6 us, 21.0 us with 4 slices)
        const int64_t tiles64 = cdiv(prob->M, 64) * cdiv(prob->N, 64);
        const int64_t tiles128 = cdiv(prob->M, 128) * cdiv(prob->N, 128);
        if (2 * tiles64 < dev->cu_count) {
            const int32_t s = slices(tiles128, 8);
            if (s >= 4) {
                want.bm = 128;
                want.bn = 128;
                want.splitk = s;
            }
        }
        // Two K slices of the 128 x 128 tiles the ladder chose when both
        // slices fit in one round and each keeps >= 16 K steps (E4M3 192 x
        // 8192 x 8192 38.6 -> 30.4 us, 512 x 4096 x 8192 39.7 -> 32.0 us,
        // 256 x 8192 x 16384 69.7 -> 50.8 us, E2M1 256 x 8192 x 16384 41.6 ->
        // 33.9 us, 384 x 4096 x 8192 23.2 -> 21.2 us; with 16 K steps or
        // fewer per slice they lose: E2M1 256 x 8192 x 4096 14.1 -> 18.6 us;
        // 4 slices lose everywhere here)
        if (want.bm == 128 && want.bn == 128 && want.splitk == 0 && 2 * tiles128 <= dev->cu_count &&
            nkt >= 32 && tiles128 <= dtg::kMaxCounters)
            want.splitk = 2;
    }
    if (force) {
        const gemm_config& f = *force;
        if (f.group_m < 0 || f.xcd_remap < 0 || f.xcd_remap > 2)
            return fail(GEMM_ERR_INVALID_ARG, "group_m must be >= 0 and xcd_remap one of 0, 1, 2");
        if ((f.kernel && f.kernel != dtg::kMxKernelTile && f.kernel != dtg::kMxKernelDirect) ||
            (f.mfma && f.mfma != 32) || f.splitk < 0 || f.splitk > 64)
            return fail(GEMM_ERR_UNSUPPORTED, "the block-scaled path runs kernels %d and %d, mfma 32, splitk 0..64",
                        dtg::kMxKernelTile, dtg::kMxKernelDirect);
        if (f.bm || f.bn || f.stages || f.waves_m || f.waves_n || f.bk || f.splitk || f.kernel) want = f;
        if (f.group_m) group_m = f.group_m;
        if (f.xcd_remap) xcd = (f.xcd_remap == GEMM_XCD_ON);
    }
    const dtg::MxEntry* e = find_entry(want, prob, *dev);
    if (!e)
        return fail(GEMM_ERR_UNSUPPORTED,
                    "no block-scaled kernel for bm=%d bn=%d bk=%d stages=%d waves=%dx%d, formats %d/%d, within "
                    "%lld bytes of LDS",
                    want.bm, want.bn, want.bk, want.stages, want.waves_m, want.waves_n, (int)prob->fmt_a,
                    (int)prob->fmt_b, (long long)dev->lds_per_wg);
    gemm_mx_plan* pl = new (std::nothrow) gemm_mx_plan;
    if (!pl) return fail(GEMM_ERR_INVALID_ARG, "out of host memory");
    pl->prob = *prob;
    pl->dev = *dev;
    pl->entry = e;
    pl->num_pid_m = cdiv(prob->M, e->bm);
    pl->num_pid_n = cdiv(prob->N, e->bn);
    const int32_t splits = want.splitk > 1 ? want.splitk : 1;
    pl->grid = pl->num_pid_m * pl->num_pid_n * splits;
    if (pl->grid > kMaxDim) {
        delete pl;
        return fail(GEMM_ERR_UNSUPPORTED, "output too large for one launch");
    }
    pl->ws_bytes = dtg::dma_workspace_bytes(pl->num_pid_m * pl->num_pid_n, e->bm, e->bn, splits);
    if (pl->ws_bytes < 0) {
        delete pl;
        return fail(GEMM_ERR_UNSUPPORTED, "K slices across workgroups support at most %d output tiles",
                    dtg::kMaxCounters);
    }
    gemm_config& c = pl->cfg;
    memset(&c, 0, sizeof c);
    c.kernel = e->kind;
    c.bm = e->bm;
    c.bn = e->bn;
    c.bk = e->bk;
    c.stages = e->stages;
    c.mfma = e->mfma;
    c.waves_m = e->waves_m;
    c.waves_n = e->waves_n;
    c.splitk = splits;
    // a band taller than the grid orders the tiles exactly as a band of the
    // whole grid: clamping keeps the kernels' band arithmetic in 32 bits
    c.group_m = static_cast<int32_t>(group_m < 1 ? 1 : group_m > pl->num_pid_m ? pl->num_pid_m : group_m);
    c.xcd_remap = (xcd && dev->xcd_count > 1) ? GEMM_XCD_ON : GEMM_XCD_OFF;
    *out = pl;
    return GEMM_OK;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

}  // namespace

extern "C" {

gemm_status gemm_mx_plan_create_for(const gemm_mx_problem* prob, const gemm_device_info* info,
                                    const gemm_config* force, gemm_mx_plan** out) {
    return plan_impl(prob, info, force, out);
}

gemm_status gemm_mx_plan_create(const gemm_mx_problem* prob, int device, const gemm_config* force,
                                gemm_mx_plan** out) {
    if (out) *out = nullptr;
    gemm_status st = validate(prob);
    if (st != GEMM_OK) return st;
    gemm_device_info info;
    st = dtg::cached_device_info(device, &info);
    if (st != GEMM_OK) return st;
    return plan_impl(prob, &info, force, out);
}

void gemm_mx_plan_destroy(gemm_mx_plan* plan) { delete plan; }

gemm_status gemm_mx_plan_config(const gemm_mx_plan* plan, gemm_config* out) {
    if (!plan || !out) return fail(GEMM_ERR_INVALID_ARG, "plan or out is NULL");
    *out = plan->cfg;
    return GEMM_OK;
}

gemm_status gemm_mx_plan_launch(const gemm_mx_plan* plan, int64_t* grid, int32_t* threads, int64_t* lds) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    if (grid) *grid = plan->grid;
    if (threads) *threads = plan->entry->threads;
    if (lds) *lds = plan->entry->lds_bytes;
    return GEMM_OK;
}

gemm_status gemm_mx_plan_describe(const gemm_mx_plan* plan, char* buf, size_t len) {
    if (!plan || !buf || len == 0) return fail(GEMM_ERR_INVALID_ARG, "plan or buf is NULL");
    const gemm_config& c = plan->cfg;
    snprintf(buf, len,
             "kernel=%s bm=%d bn=%d bk=%d stages=%d mfma=%d waves=%dx%d group_m=%d splitk=%d xcd_remap=%d "
             "grid=%lld threads=%d lds=%lld fmt=%d/%d out=%d",
             plan->entry->name, c.bm, c.bn, c.bk, c.stages, c.mfma, c.waves_m, c.waves_n, c.group_m, c.splitk,
             c.xcd_remap, (long long)plan->grid, plan->entry->threads, (long long)plan->entry->lds_bytes,
             (int)plan->prob.fmt_a, (int)plan->prob.fmt_b, (int)plan->prob.out);
    return GEMM_OK;
}

gemm_status gemm_mx_workspace_size(const gemm_mx_plan* plan, size_t* bytes) {
    if (!plan || !bytes) return fail(GEMM_ERR_INVALID_ARG, "plan or bytes is NULL");
    *bytes = static_cast<size_t>(plan->ws_bytes);
    return GEMM_OK;
}

gemm_status gemm_mx_workspace_init(const gemm_mx_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    if (plan->ws_bytes == 0) return GEMM_OK;
    if (!workspace || workspace_bytes < static_cast<size_t>(plan->ws_bytes))
        return fail(GEMM_ERR_WORKSPACE, "workspace of %zu bytes given, %lld needed", workspace_bytes,
                    (long long)plan->ws_bytes);
    hipError_t e = dtg::zero_words(workspace, plan->ws_bytes / 4, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GEMM_ERR_HIP, "workspace zero fill: %s", hipGetErrorString(e));
    return GEMM_OK;
}

gemm_status gemm_mx_run(const gemm_mx_plan* plan, const void* A, const void* SA, const void* B, const void* SB,
                        const void* C, void* D, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(GEMM_ERR_INVALID_ARG, "plan is NULL");
    const gemm_mx_problem& p = plan->prob;
    if (p.has_c && !C) return fail(GEMM_ERR_INVALID_ARG, "problem has C but C is NULL");
    if (!p.has_c && C) return fail(GEMM_ERR_INVALID_ARG, "C given but the problem has has_c = 0");
    if (p.M == 0 || p.N == 0) return GEMM_OK;
    if (!D) return fail(GEMM_ERR_INVALID_ARG, "D is NULL");
    const int esz = p.out == GEMM_MX_OUT_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(D) % esz || (C && reinterpret_cast<uintptr_t>(C) % esz))
        return fail(GEMM_ERR_UNSUPPORTED, "C and D must be aligned to their element size");
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(D);
    const uintptr_t d1 = d0 + static_cast<uintptr_t>(((p.M - 1) * p.ldd + p.N) * esz);
    if (p.K > 0) {
        if (!A || !B || !SA || !SB) return fail(GEMM_ERR_INVALID_ARG, "A, SA, B or SB is NULL");
        if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(B) & 15))
            return fail(GEMM_ERR_UNSUPPORTED, "A and B must be 16-byte aligned");
        if ((reinterpret_cast<uintptr_t>(SA) & 3) || (reinterpret_cast<uintptr_t>(SB) & 3))
            return fail(GEMM_ERR_UNSUPPORTED, "SA and SB must be 4-byte aligned");
        const struct { const void* ptr; int64_t bytes; const char* name; } in[4] = {
            {A, (p.M - 1) * p.lda + row_bytes(p.K, p.fmt_a), "A"},
            {B, (p.N - 1) * p.ldb + row_bytes(p.K, p.fmt_b), "B"},
            {SA, p.M * p.ldsa, "SA"},
            {SB, p.N * p.ldsb, "SB"}};
        for (const auto& x : in) {
            const uintptr_t x0 = reinterpret_cast<uintptr_t>(x.ptr);
            if (overlaps(d0, d1, x0, x0 + static_cast<uintptr_t>(x.bytes)))
                return fail(GEMM_ERR_INVALID_ARG, "D overlaps %s", x.name);
        }
    }
    if (p.has_c) {
        const uintptr_t c0 = reinterpret_cast<uintptr_t>(C);
        const uintptr_t c1 = c0 + static_cast<uintptr_t>(((p.M - 1) * p.ldc + p.N) * esz);
        const bool same = (C == D) && (p.ldc == p.ldd || p.M == 1);
        if (!same && overlaps(d0, d1, c0, c1))
            return fail(GEMM_ERR_INVALID_ARG, "D overlaps C (only D == C with equal strides is allowed)");
    }
    if (plan->ws_bytes > 0) {
        if (!workspace || workspace_bytes < static_cast<size_t>(plan->ws_bytes))
            return fail(GEMM_ERR_WORKSPACE, "plan needs a workspace of %lld bytes (%zu given)",
                        (long long)plan->ws_bytes, workspace ? workspace_bytes : static_cast<size_t>(0));
        if (reinterpret_cast<uintptr_t>(workspace) & 255)
            return fail(GEMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    dtg::MxArgs a;
    a.A = static_cast<const uint8_t*>(A);
    a.B = static_cast<const uint8_t*>(B);
    a.SA = static_cast<const uint8_t*>(SA);
    a.SB = static_cast<const uint8_t*>(SB);
    a.C = C;
    a.D = D;
    a.M = static_cast<int32_t>(p.M);
    a.N = static_cast<int32_t>(p.N);
    a.K = static_cast<int32_t>(p.K);
    a.num_pid_m = static_cast<int32_t>(plan->num_pid_m);
    a.num_pid_n = static_cast<int32_t>(plan->num_pid_n);
    a.group_m = plan->cfg.group_m;
    a.xcds = (plan->cfg.xcd_remap == GEMM_XCD_ON) ? plan->dev.xcd_count : 1;
    a.has_c = p.has_c;
    a.out = static_cast<int32_t>(p.out);
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldsa = p.ldsa;
    a.ldsb = p.ldsb;
    a.ldc = p.has_c ? p.ldc : 0;
    a.ldd = p.ldd;
    a.splits = plan->cfg.splitk;
    a.ws = workspace;
    hipError_t err = plan->entry->launch(a, plan->grid, static_cast<hipStream_t>(stream));
    if (err != hipSuccess)
        return fail(GEMM_ERR_HIP, "launch of %s: %s", plan->entry->name, hipGetErrorString(err));
    return GEMM_OK;
}

}  // extern "C"
