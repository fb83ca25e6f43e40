// Skinny-M GEMM kernel for gfx950:  D = A x B (+ C) with M <= 32.
//
// With a handful of rows the product is bound by streaming B from HBM (the
// decode regime of "Tuning Triton", section 4: a skinny M wants its own tile
// family, BM = 16 with a deep K).  K is split twice ("Tuning Triton", section
// 6: a K split is the axis that matters at M = 16; "Hopper Support in
// Triton", slides 15-16: SPLIT_K): across S workgroups per BN-column slab of D
// (S is a launch parameter) and, inside a workgroup, across its NWV waves.
// HBM streams well only when each workgroup reads at least a 128-byte band of
// every row of B, so slabs are 64 or 128 columns wide and S supplies the
// parallelism (N = 8192, BN = 128, S = 4: 256 workgroups).
// Each wave streams its K range in CK-deep chunks through a private ST-stage
// LDS ring with direct global -> LDS loads (B rows of BN columns, A rows of
// CK k), so no workgroup barrier is needed until the end; the A operand is
// read with 16-byte LDS reads and the B operand with the transposing 64-bit
// LDS read, and one v_mfma_f32_16x16x32 per 16 columns per 32 k accumulates
// in fp32.  The NWV partial 16 x BN tiles are then summed through LDS in a
// fixed wave order.  With S = 1 the workgroup then adds C in fp32, rounds and
// stores rows < M, columns < N.  With S > 1 it writes its fp32 partial tile to
// the workspace and counts itself in on the slab's counter; the workgroup that
// arrives last sums the S partials in slice order (so the result does not
// depend on arrival order), adds C, rounds, stores, and resets the counter to
// zero for the next launch.  The counters sit in a fixed region at the head of
// the workspace, so one zero-filled workspace serves every plan in turn.
//
// Out-of-range rows of A (>= M), columns of B (>= N) and k (>= K) are loaded
// as zeros through buffer offsets past the descriptor range.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace dtg {
namespace {

using namespace dev;

// B stage layout: CK rows of BN contiguous columns.  One transposing read
// touches rows 8 g + 4 h + 0..3 for lane groups g; these layouts keep the
// rows of groups g and g + 1 in different banks:
//  BN = 32 (64-byte rows): the two 32-byte halves of a row swap when bit 3
//          of the row index is set;
//  BN = 16 (32-byte rows): rows 8..15 of every 16 are stored in the order
//          12..15, 8..11 (row r sits at position r ^ (4 * bit 3 of r));
//  BN = 64 (128-byte rows): chunk pairs XOR 2 * (bit 1 of r | bit 3 of r << 1),
//          so the 8 rows two neighbouring lane groups read tile one 256-byte
//          bank window;
//  BN = 128, 256 (256-, 512-byte rows): chunk pairs XOR 2 * ((r & 3) | bit 3
//          of r << 2).
// All these maps are involutions.
// The workspace starts with the fixed region of kMaxCounters arrival counters, the
// same for every plan, so plans of any slab count can share one workspace;
// fp32 partial tiles follow.

template <int BN>
__device__ __forceinline__ int b_pos(int r) {
    if constexpr (BN == 16) return r ^ (((r >> 3) & 1) << 2);
    else return r;
}
template <int BN>
__device__ __forceinline__ int b_chunk(int r, int q) {
    if constexpr (BN == 32) return q ^ (((r >> 3) & 1) << 1);
    else if constexpr (BN == 64) return q ^ (2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)));
    else if constexpr (BN >= 128) return q ^ (2 * ((r & 3) | (((r >> 3) & 1) << 2)));
    else return q;
}

// BMR: rows of the output slab (16 or 32: one or two 16-row MFMA blocks).
template <int BN, int NWV, int CK, int ST, bool BF16, int BMR>
__global__ __launch_bounds__(64 * NWV) void gemm_skinny_kernel(KArgs p) {
    constexpr int NT = 64 * NWV;
    constexpr int CHB = BN / 8;            // 16-byte chunks per B row
    constexpr int RB = 64 / CHB;           // B rows per wave instruction
    constexpr int IB = CK / RB;            // B instructions per chunk
    constexpr int CHA = CK / 8;            // 16-byte chunks per A row
    constexpr int RA = 64 / CHA;           // A rows per wave instruction
    constexpr int IA = BMR / RA;           // A instructions per chunk
    constexpr int MB = BMR / 16;           // 16-row MFMA blocks
    constexpr int FN = BN / 16;
    constexpr int KSN = CK / 32;
    constexpr int SB = CK * BN, SAE = BMR * CK, STG = SB + SAE;  // elements
    constexpr int OPS = IB + IA;           // vector-memory ops per chunk
    static_assert(BN == 16 || BN == 32 || BN == 64 || BN == 128 || BN == 256, "BN");
    static_assert(CK == 32 || CK == 64, "CK");
    static_assert(IA >= 1 && IB >= 1, "load split");
    static_assert(ST >= 2 && ST <= 8 && (ST - 2) * OPS < 64, "stages");
    static_assert(BMR == 16 || BMR == 32, "BMR");
    static_assert(NWV * ST * STG * 2 >= NWV * BMR * BN * 4 + 4, "reduction buffer and flag");
    static_assert(OPS < 64, "vmcnt");

    __shared__ __attribute__((aligned(1024))) uint16_t smem[NWV * ST * STG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup -> (slab, slice): consecutive positions are consecutive slabs of
    // one slice, and the XCD permutation gives each die one contiguous run of
    // positions, so a die's L2 sees whole rows of a band of columns.
    const int nslabs = p.num_pid_n;
    const int S = p.splits;
    const int pos = xcd_permute<int>(blockIdx.x, gridDim.x, p.xcds);
    const int slab = pos % nslabs, slice = pos / nslabs;
    const int M = p.M, N = p.N, K = p.K;
    // Columns of the slab: its first and second halves start at colx and
    // coly.  A 128-column slab of a whole run of 512 columns (1 KiB of a row)
    // takes 64-column blocks 0 and 2, 1 and 3, 4 and 6 or 5 and 7 of the run
    // rather than two adjacent ones, so that each workgroup reads two
    // different 256-byte quarters of every 1 KiB (slabs that read only the
    // second quarter of each 1 KiB were measured to finish last): 16 x 8192
    // x 8192 31.0 -> 30.5 us, bitwise the same.  Otherwise the slab is BN
    // contiguous columns.
    int colx = slab * BN, coly = slab * BN + BN / 2;
    if constexpr (BN == 128) {
        const int grp = slab / 4, i = slab % 4;
        if (grp * 512 + 512 <= N) {
            colx = grp * 512 + ((i < 2) ? i : i + 2) * 64;
            coly = colx + 128;
        }
    }
    auto real_col = [&](int c) { return c < BN / 2 ? colx + c : coly + (c - BN / 2); };

    // chunks of this slice, then of this wave
    const int nck = (K + CK - 1) / CK;
    const int per_slice = (nck + S - 1) / S;
    const int s_first = slice * per_slice;
    const int s_end = (s_first + per_slice < nck) ? s_first + per_slice : nck;
    const int s_n = s_end > s_first ? s_end - s_first : 0;
    const int per = (s_n + NWV - 1) / NWV;
    const int c_first = s_first + wave * per;
    const int c_last = (wave * per + per < s_n) ? c_first + per : s_first + s_n;
    const int nc = c_last > c_first ? c_last - c_first : 0;

    // ---- per-lane load offsets (bytes from the per-chunk descriptors)
    uint32_t b_voff[IB];
    int b_row[IB];
    bool b_ok[IB];
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        const int pos = i * RB + lane / CHB;
        const int r = b_pos<BN>(pos);
        const int q = b_chunk<BN>(r, lane % CHB);
        b_row[i] = r;
        b_ok[i] = real_col(8 * q) < N;
        b_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * p.ldb * 2 + real_col(8 * q) * 2);
    }
    uint32_t a_voff[IA];
    int a_kc[IA];
    bool a_ok[IA];
#pragma unroll
    for (int i = 0; i < IA; ++i) {
        const int row = i * RA + lane / CHA;
        const int q = (lane % CHA) ^ swz<CHA>(row);
        a_ok[i] = row < M;
        a_kc[i] = 8 * q;
        a_voff[i] = static_cast<uint32_t>(static_cast<int64_t>(row) * p.lda * 2 + q * 16);
    }

    // Slabs of 128 or more columns walk their chunks starting at a rotation
    // set by the slab's 512-column run g (1 KiB of a row), chunk 3 g mod nc
    // first, so that at any moment the runs read different rows of B rather
    // than all the same ones: with B from HBM, 1 and 16 x 8192 x 8192
    // 29.2-29.4 -> 28.2-28.6 us (g mod nc, or per 256 columns, gained less);
    // the narrower slabs lose by it (64 columns at 4096 x 4096: 11.5 -> 12.3
    // us) and keep the plain order.  A run's slabs share the rotation, so
    // slabs of 128 and 256 columns with equal K partitions still agree bit
    // for bit.
    const int rot = (BN >= 128 && nc > 0) ? ((colx >> 9) * 3) % nc : 0;
    auto issue = [&](int c, int slot) {
        const int cr = c + rot;   // chunks in the order rot, rot + 1, ..., nc - 1, 0, ..., rot - 1
        const int k0 = (c_first + (cr >= nc ? cr - nc : cr)) * CK;
        const uint16_t* bbase = p.B + static_cast<int64_t>(k0) * p.ldb;
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(bbase), 0,
            clamp_records((static_cast<int64_t>(K - 1 - k0) * p.ldb + N) * 2), kRsrcWord3);
        const uint16_t* abase = p.A + k0;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(abase), 0,
            clamp_records((static_cast<int64_t>(M - 1) * p.lda + (K - k0)) * 2), kRsrcWord3);
        uint16_t* sb = smem + (wave * ST + slot) * STG;
        uint16_t* sa = sb + SB;
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            const uint32_t v = (b_ok[i] && k0 + b_row[i] < K) ? b_voff[i] : kOOB;
            // B is read exactly once: non-temporal loads (16 x 8192 x 8192 from
            // HBM 28.4 -> 27.0 us, 1 x 4096 x 4096 11.3 -> 11.0, 1 x 2048 x 2048
            // 7.05 -> 6.85; A, shared by every slab, keeps the default policy)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(sb + i * 512), 16, v, 0, 0, kNonTemporal);
        }
#pragma unroll
        for (int i = 0; i < IA; ++i) {
            const uint32_t v = (a_ok[i] && k0 + a_kc[i] < K) ? a_voff[i] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sa + i * 512), 16, v, 0, 0, 0);
        }
    };

    // ---- per-lane operand read offsets (LDS bytes within a stage)
    uint32_t a_off[MB][KSN], b_off[FN][KSN][2];
    {
        const int g = lane >> 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int i = mb * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
                a_off[mb][ks] = (SB + i * CK + (((ks * 4 + g) ^ swz<CHA>(i)) * 8)) * 2;   // chunk ks*4 + g of row i
        }
        const int jq = lane & 15;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = ks * 32 + 8 * g + 4 * h + (jq >> 2);
                    const int col = fn * 16 + 4 * (jq & 3);
                    const int ph = b_chunk<BN>(r, col >> 3);
                    b_off[fn][ks][h] = (b_pos<BN>(r) * BN + ph * 8 + (col & 7)) * 2;
                }
    }

    f32x4 acc[MB][FN];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[mb][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const uint32_t ring = lds_addr(smem) + wave * ST * STG * 2;
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
        if (s < nc) issue(s, s);
    for (int c = 0; c < nc; ++c) {
        // chunk c is complete once at most the chunks issued after it remain
        // in flight: min(ST - 2, nc - 1 - c) chunks of OPS loads each
        const int after = (nc - 1 - c < ST - 2) ? (nc - 1 - c) : (ST - 2);
        static_for<ST - 1>([&](auto i_tag) {
            constexpr int I = decltype(i_tag)::value;
            if (after == I) wait_vm<I * OPS>();
        });
        const int slot = c % ST;
        if (c + ST - 1 < nc) issue(c + ST - 1, (c + ST - 1) % ST);
        const uint32_t base = ring + slot * STG * 2;
        u32x4 af[MB][KSN], bf[FN][KSN];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) af[mb][ks] = lds_read16<0>(base + a_off[mb][ks]);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                const i16x4 h0 = lds_read_tr<0>(base + b_off[fn][ks][0]);
                const i16x4 h1 = lds_read_tr<0>(base + b_off[fn][ks][1]);
                bf[fn][ks] = __builtin_bit_cast(u32x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        lds_wait_all();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) tie(af[mb][ks]);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) tie(bf[fn][ks]);
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) acc[mb][fn] = mfma<16, BF16>(af[mb][ks], bf[fn][ks], acc[mb][fn]);
    }

    // ---- sum the wave partials in a fixed order, + C, round, store
    __syncthreads();                                   // every ring is drained
    float* red = reinterpret_cast<float*>(smem);       // [NWV][BMR][BN]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(wave * BMR + mb * 16 + 4 * (lane >> 4) + r) * BN + fn * 16 + (lane & 15)] = acc[mb][fn][r];
    __syncthreads();
    const bool has_c = p.has_c != 0;
    if (S == 1) {
        for (int t = tid; t < BMR * BN; t += NT) {
            const int row = t / BN, col = t % BN;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NWV; ++w) v += red[(w * BMR + row) * BN + col];
            const int gc = real_col(col);
            if (row < M && gc < N) {
                if (has_c) v += widen<BF16>(p.C[static_cast<int64_t>(row) * p.ldc + gc]);
                p.D[static_cast<int64_t>(row) * p.ldd + gc] = narrow<BF16>(v);
            }
        }
        return;
    }
    // ---- S > 1: partial tile -> workspace; the last workgroup of the slab sums.
    // The partials are written and read with system-scope atomic accesses,
    // which go past the (per-XCD, mutually non-coherent) L2 caches to memory;
    // see arrive_last for the ordering.
    int* counters = static_cast<int*>(p.ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(p.ws) + kCounterBytes) +
                  static_cast<int64_t>(slab) * S * BMR * BN;
    // Each thread owns runs of 4 consecutive outputs of one row (16 bytes of
    // partial): 16-byte LDS reads of the wave partials, one 16-byte
    // system-coherent store of its slice's partial, one 16-byte load per other
    // slice.  Summation order as ever: waves 0..NWV-1, then slices 0..S-1.
    constexpr int RUNS = BMR * BN / 4;                // 4-output runs of the tile
    constexpr int PR = (RUNS + NT - 1) / NT;          // runs per thread
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, clamp_records(static_cast<int64_t>(S) * BMR * BN * 4), kRsrcWord3);
    f32x4 mine[PR];
#pragma unroll
    for (int j = 0; j < PR; ++j) {
        const int t = 4 * (tid + j * NT);
        mine[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (t >= BMR * BN) break;
#pragma unroll
        for (int w = 0; w < NWV; ++w) mine[j] += *reinterpret_cast<const f32x4*>(&red[w * BMR * BN + t]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[j]), pr,
                                               static_cast<uint32_t>((slice * BMR * BN + t) * 4), 0, kSysScope);
    }
    // the arrival flag lives just past the wave partials
    if (!arrive_last(&counters[slab], S, reinterpret_cast<int*>(red + NWV * BMR * BN))) return;
    // The other slices' partials are loaded in groups of up to 8 slices, all at
    // once, then summed in slice order; this slice's own comes from registers
    // (bitwise the value it stored).
    f32x4 v[PR];
#pragma unroll
    for (int j = 0; j < PR; ++j) v[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += 8) {
        f32x4 x[8][PR];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < PR; ++j) {
                const int t = 4 * (tid + j * NT);
                const bool other = s0 + u < S && s0 + u != slice && t < BMR * BN;
                x[u][j] = other ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                pr, static_cast<uint32_t>(((s0 + u) * BMR * BN + t) * 4),
                                                                0, kSysScope))
                                : mine[j];
            }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < PR; ++j)
                if (s0 + u < S) v[j] += x[u][j];
    }
#pragma unroll
    for (int j = 0; j < PR; ++j) {
        const int t = 4 * (tid + j * NT);
        const int row = t / BN, col = t % BN;
        const int gc = real_col(col);             // 4 consecutive columns (a run never crosses a half slab)
        if (t < BMR * BN && row < M && gc < N) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (gc + e >= N) break;
                float o = v[j][e];
                if (has_c) o += widen<BF16>(p.C[static_cast<int64_t>(row) * p.ldc + gc + e]);
                p.D[static_cast<int64_t>(row) * p.ldd + gc + e] = narrow<BF16>(o);
            }
        }
    }
    if (tid == 0) __hip_atomic_store(&counters[slab], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int BN, int NWV, int CK, int ST, bool BF16, int BMR>
hipError_t launch_skinny(const KArgs& a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_skinny_kernel<BN, NWV, CK, ST, BF16, BMR>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * NWV), 0, stream, a);
    return hipGetLastError();
}

#define DTG_STR2(x) #x
#define DTG_STR(x) DTG_STR2(x)
#define SKINNY_ENTRY(BN, NWV, CK, ST, BF, BMR)                                               \
    {KF_SKINNY, BMR, BN, CK, ST, 16, 1, NWV, 0, BF, 1, 64 * NWV,                            \
     static_cast<int64_t>(NWV) * ST * (CK * BN + BMR * CK) * 2,                             \
     &launch_skinny<BN, NWV, CK, ST, (BF != 0), BMR>,                                       \
     "gemm_skinny_kernel<" DTG_STR(BN) "," DTG_STR(NWV) "," DTG_STR(CK) "," DTG_STR(ST) ","  \
     DTG_STR(BF) "," DTG_STR(BMR) ">", 0}
#define SKINNY_BOTH(BN, NWV, CK, ST) SKINNY_ENTRY(BN, NWV, CK, ST, 0, 16), SKINNY_ENTRY(BN, NWV, CK, ST, 1, 16)
#define SKINNY32_BOTH(BN, NWV, CK, ST) SKINNY_ENTRY(BN, NWV, CK, ST, 0, 32), SKINNY_ENTRY(BN, NWV, CK, ST, 1, 32)

const KernelEntry kSkinnyTable[] = {
    SKINNY_BOTH(256, 4, 32, 2),
    SKINNY_BOTH(128, 4, 32, 3),
    SKINNY_BOTH(128, 4, 32, 4),
    SKINNY_BOTH(128, 2, 32, 8),
    SKINNY_BOTH(128, 2, 32, 6),
    SKINNY_BOTH(128, 8, 32, 2),
    SKINNY_BOTH(64, 4, 64, 3),
    SKINNY_BOTH(64, 8, 64, 2),
    SKINNY_BOTH(32, 8, 64, 3),
    SKINNY_BOTH(16, 8, 64, 3),
    SKINNY32_BOTH(128, 8, 32, 2),
    SKINNY32_BOTH(128, 4, 32, 3),
    SKINNY32_BOTH(64, 8, 32, 3),
    SKINNY32_BOTH(32, 8, 32, 3),
};

}  // namespace

namespace {
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = 0u;
}
}  // namespace

hipError_t zero_words(void* p, int64_t nwords, hipStream_t stream) {
    if (nwords <= 0) return hipSuccess;
    const int64_t blocks = (nwords + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(p), nwords);
    return hipGetLastError();
}

int64_t skinny_workspace_bytes(int64_t nslabs, int bm, int bn, int splits) {
    if (splits <= 1) return 0;
    if (nslabs > kMaxCounters) return -1;
    return kCounterBytes + nslabs * splits * static_cast<int64_t>(bm) * bn * 4;
}

const KernelEntry* skinny_kernel_table(int* count) {
    *count = static_cast<int>(sizeof(kSkinnyTable) / sizeof(kSkinnyTable[0]));
    return kSkinnyTable;
}

}  // namespace dtg
