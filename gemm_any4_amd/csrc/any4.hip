// libany4 -- any4 dequantize-GEMM for MI355X (gfx950, CDNA4).
//
// What is computed (the 10100.com any4 explainer): each weight is a 4-bit index
// into its row's 16-entry bf16 table (section 二), each contiguous group of g
// weights of a row has a scale alpha and an offset beta (step 1, "分组缩放"), so
// w = alpha * LUT_row[idx] + beta; the matmul y = x * W^T runs at decode batch
// sizes 1..16 (section 三).  The C ABI is declared in include/any4.h.
//
// Packed tile layout (written by k_pack, read by k_dequant and k_gemm)
//   The weights are cut into tiles of 16 rows x 128 k.  A tile is 1 KB and is
//   one 16-byte load per lane of a wave64: lane l holds row (l % 16) of the
//   tile, k in [32*(l/16), 32*(l/16) + 32), two indices per byte, the even k
//   in the low nibble.  Tiles are stored row-block major: tile (b, c) of row
//   block b (rows 16b..16b+15) and k-chunk c (k 128c..128c+127) starts at byte
//   (b * K/128 + c) * 1024.  Rows past N are zero padding.
//
// Kernels
//   k_pack     idx[N][K] u8 -> tiles, 16 output bytes per thread.
//   k_dequant  w = bf16(fma(alpha, LUT[idx], beta)), one tile slot per thread.
//   k_gemm     y = x * W^T with v_mfma_f32_16x16x32_bf16; see the comment above
//              the kernel.
#include <hip/hip_runtime.h>

#include "any4.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int TILE_ROWS = 16;
constexpr int TILE_K = 128;
constexpr int TILE_BYTES = TILE_ROWS * TILE_K / 2;   // 1024

__device__ __forceinline__ float bf16_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ---------------------------------------------------------------------------
// bounds-checked buffer loads
// ---------------------------------------------------------------------------
constexpr uint32_t OOR = 0x80000000u;   // an offset past every buffer this library reads

// Raw buffer resource over [base, base + bytes): a load at an offset >= bytes
// returns zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// pack
// ---------------------------------------------------------------------------
constexpr int PACK_THREADS = 256;

// Two dwords of indices (bytes i0..i7) -> one dword (i0|i1<<4, i2|i3<<4, i4|i5<<4, i6|i7<<4).
__device__ __forceinline__ uint32_t pack8(uint32_t lo4, uint32_t hi4)
{
    uint32_t t = lo4 & 0x0F0F0F0Fu;
    uint32_t u = hi4 & 0x0F0F0F0Fu;
    t |= t >> 4;   // byte 0 = i0 | i1 << 4, byte 2 = i2 | i3 << 4
    u |= u >> 4;
    return __builtin_amdgcn_perm(u, t, 0x06040200u);
}

// One thread per 16-byte tile slot: tile q/64, lane q%64.
__global__ __launch_bounds__(PACK_THREADS) void k_pack(const uint8_t* __restrict__ idx,
                                                       uint8_t* __restrict__ packed, int N,
                                                       int K, uint32_t slots)
{
    const uint32_t q = blockIdx.x * PACK_THREADS + threadIdx.x;
    if (q >= slots)
        return;
    const int Kc = K / TILE_K;
    const uint32_t tile = q >> 6, l = q & 63;
    const int b = tile / Kc, c = tile % Kc;
    const int n = b * TILE_ROWS + (l & 15);
    u32x4_t out = {0u, 0u, 0u, 0u};
    if (n < N) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
            idx + static_cast<size_t>(n) * K + c * TILE_K + (l >> 4) * 32);
        const u32x4_t a = src[0], bb = src[1];
        out[0] = pack8(a[0], a[1]);
        out[1] = pack8(a[2], a[3]);
        out[2] = pack8(bb[0], bb[1]);
        out[3] = pack8(bb[2], bb[3]);
    }
    *reinterpret_cast<u32x4_t*>(packed + static_cast<size_t>(q) * 16) = out;
}

// ---------------------------------------------------------------------------
// dequant
// ---------------------------------------------------------------------------
constexpr int DQ_WAVES = 4;   // one tile per wave; a workgroup covers 4 chunks of one row block

// w[n][k] = bf16(fma(alpha, LUT[idx], beta)).  The workgroup's 16 table rows
// are widened to fp32 in LDS; each lane decodes its 32 weights and writes 64
// contiguous bytes of w.
__global__ __launch_bounds__(64 * DQ_WAVES) void k_dequant(const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ lut,
                                                          const uint16_t* __restrict__ alpha,
                                                          const uint16_t* __restrict__ beta,
                                                          uint16_t* __restrict__ w, int N, int K,
                                                          int g)
{
    __shared__ float sl[TILE_ROWS * 16];
    const int Kc = K / TILE_K;
    const int cgroups = (Kc + DQ_WAVES - 1) / DQ_WAVES;
    const int b = blockIdx.x / cgroups;
    const int c = (blockIdx.x % cgroups) * DQ_WAVES + (threadIdx.x >> 6);
    {
        const int t = threadIdx.x;   // 256 threads: row t/16, entry t%16
        const int n = b * TILE_ROWS + (t >> 4);
        sl[t] = n < N ? bf16_to_f32(lut[static_cast<size_t>(n) * 16 + (t & 15)]) : 0.f;
    }
    __syncthreads();
    const int l = threadIdx.x & 63;
    const int j = l & 15;
    const int n = b * TILE_ROWS + j;
    if (c >= Kc || n >= N)
        return;
    const int k0 = c * TILE_K + (l >> 4) * 32;
    const int G = K / g;
    const float a = bf16_to_f32(alpha[static_cast<size_t>(n) * G + k0 / g]);
    const float bt = bf16_to_f32(beta[static_cast<size_t>(n) * G + k0 / g]);
    const u32x4_t p = *reinterpret_cast<const u32x4_t*>(
        packed + (static_cast<size_t>(b) * Kc + c) * TILE_BYTES + l * 16);
    const float* L = sl + j * 16;
    u32x4_t out[4];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t byte = (p[q >> 2] >> (8 * (q & 3))) & 0xFFu;
        const float lo = fmaf(a, L[byte & 15u], bt);
        const float hi = fmaf(a, L[byte >> 4], bt);
        out[q >> 2][q & 3] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(w + static_cast<size_t>(n) * K + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        dst[q] = out[q];
}

// ---------------------------------------------------------------------------
// gemm
// ---------------------------------------------------------------------------

// y = 0 (the K = 0 case: every sum is empty).  A kernel rather than a memset,
// so that the call can be captured in a HIP graph.
__global__ __launch_bounds__(256) void k_zero(uint16_t* __restrict__ y, size_t n)
{
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n)
        y[i] = 0;
}

// Work split.  A workgroup has 8 waves and stays resident for the whole call
// (the grid is about one workgroup per CU).  K is cut into S parts of 8*C
// chunks; wave w of a workgroup always works on the same C chunks of its
// part, so the x operands of those chunks are loaded once, into VGPRs, and
// reused for every row block.  The workgroup walks row blocks r, r+Gp, r+2Gp,
// ... (Gp workgroups per part); for each block its 8 waves decode their chunks
// and their partial sums meet in LDS.  With S > 1 the parts of a block are
// summed by whichever workgroup finishes that block last (counter in the
// workspace), in part order, so results do not depend on timing.
//
// Decode.  A packed byte (two indices) selects one dword of a pair table in
// LDS: entry (hi << 4 | lo) holds (LUT[lo], LUT[hi]) as two bf16, which is
// exactly one dword of an MFMA B operand.  The table of a row block has 32
// slots per entry (slot = lane % 32, row = slot % 16); a wave64 LDS read is
// served as two halves of 32 lanes, so every lane reads its own bank: no
// conflicts.  Entry e of buffer q sits at byte e*256 + q*128, so the read
// address is one v_perm of the packed dword.  Two buffers let the waves build
// the next block's table while they decode the current one.
//
// Scale and offset.  Per 128-k chunk a lane accumulates sum_k x*LUT[idx] with
// four MFMAs, then adds alpha times that sum and beta times sum_k x (the chunk
// sums of x are computed once, with MFMAs against ones).
//
// Memory.  Each wave keeps the next D tiles of its sequence (plus their alpha
// and beta) in flight in a register ring, and loads the tables LR blocks
// ahead.  Every load is a bounds-checked buffer load; where there is nothing
// to read (past the wave's work, x rows m >= M) its offset is pushed out of
// range, so no branch guards a load and no traffic is made.
constexpr int GW = 8;                   // waves per workgroup
constexpr int GT = 64 * GW;
constexpr int TAB_BYTES = 256 * 256;    // 256 entries x 2 buffers x 32 slots x 4 B
constexpr int RED_BYTES = 2 * GW * 64 * 16;

struct GemmArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* lut;
    const uint16_t* alpha;
    const uint16_t* beta;
    uint16_t* y;
    float* part;        // [S][NB][64][VC] partial sums (S > 1)
    uint32_t* count;    // [NB] arrival counters, zero between calls (S > 1)
    int M, N, K, g;
    int S, Gp;
};

// Byte address of table entry `byte j of d` in the lane's slot: (d.byte[j] << 8) | slot4.
__device__ __forceinline__ uint32_t tab_addr(uint32_t d, uint32_t slot4, int j)
{
    return __builtin_amdgcn_perm(d, slot4, 0x0C0C0000u | ((4u + j) << 8));
}

__device__ __forceinline__ uint32_t lds_word(const uint8_t* smem, uint32_t byte_addr)
{
    return *reinterpret_cast<const uint32_t*>(smem + byte_addr);
}

template <int MT, int C, int D, int LR>
__global__ __launch_bounds__(GT) void k_gemm(const GemmArgs args)
{
    static_assert(D % C == 0 && (D / C) % LR == 0, "ring sizes");
    __shared__ __attribute__((aligned(16))) uint8_t smem[TAB_BYTES + RED_BYTES];
    constexpr int VC = MT < 4 ? MT : 4;   // accumulator rows that can hold a real m

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;      // tile row of this lane (B operand), x row m (A operand)
    const int kq = lane >> 4;     // 32-k quarter of a chunk
    const int Kc = K / TILE_K;
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = K / g;
    const int s = blockIdx.x / args.Gp;
    const int r = blockIdx.x % args.Gp;
    const int nblk = r < NB ? (NB - 1 - r) / args.Gp + 1 : 0;
    const int T = nblk * C;                 // tiles in this wave's sequence
    const int cbase = s * (GW * C) + wave * C;

    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TILE_BYTES);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, static_cast<uint32_t>(N) * 32);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, static_cast<uint32_t>(N) * G * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, static_cast<uint32_t>(N) * G * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // ---- table rows: thread tid builds slot st (row st % 16), entries lo + 16*hi
    const int st = tid & 31;
    const int lo = tid >> 5;   // 0..15
    u32x4_t lq0[LR], lq1[LR];
    uint32_t llo[LR];
    auto lut_load = [&](int i, u32x4_t& q0, u32x4_t& q1, uint32_t& ll) {
        const uint32_t row = static_cast<uint32_t>(r + i * args.Gp) * TILE_ROWS + (st & 15);
        const uint32_t off = i < nblk ? row * 32u : OOR;
        q0 = load16(rl, off);
        q1 = load16(rl, off + 16);
        ll = load2(rl, off + 2 * lo);
    };
    auto tab_build = [&](int buf, const u32x4_t& q0, const u32x4_t& q1, uint32_t ll) {
        const uint32_t Lw[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        uint32_t* tw = reinterpret_cast<uint32_t*>(smem) + lo * 64 + buf * 32 + st;
#pragma unroll
        for (int hi = 0; hi < 16; ++hi)
            tw[hi * 16 * 64] = __builtin_amdgcn_perm(Lw[hi >> 1], ll,
                                                     (hi & 1) ? 0x07060100u : 0x05040100u);
    };

    // ---- tile ring
    u32x4_t pb[D];
    uint32_t ab[D], bbv[D];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * 16;
    auto issue = [&](int u, int t) {
        const int i = t / C;
        const int c = cbase + t % C;
        const bool live = t < T && c < Kc;
        const int b = r + i * args.Gp;
        const uint32_t toff = static_cast<uint32_t>(b * Kc + c) * TILE_BYTES + tile_lane;
        const uint32_t goff =
            (static_cast<uint32_t>(b * TILE_ROWS + j) * G + (c * TILE_K) / g) * 2;
        pb[u] = load16(rp, live ? toff : OOR);
        ab[u] = load2(ra, live ? goff : OOR);
        bbv[u] = load2(rb, live ? goff : OOR);
    };

    // ---- prologue: table of block 0, x operands, the first D tiles, tables 1..LR
    lut_load(0, lq0[0], lq1[0], llo[0]);
    u32x4_t xr[C][4];
#pragma unroll
    for (int ci = 0; ci < C; ++ci) {
        const int c = cbase + ci;
        const bool live = j < M && c < Kc;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
            xr[ci][s4] = load16(rx, live ? static_cast<uint32_t>(
                                               (j * K + c * TILE_K + kq * 32 + s4 * 8) * 2)
                                         : OOR);
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
        issue(u, u);
    tab_build(0, lq0[0], lq1[0], llo[0]);
#pragma unroll
    for (int q = 1; q <= LR; ++q)
        lut_load(q, lq0[q % LR], lq1[q % LR], llo[q % LR]);

    // chunk sums of x: lane l gets sum_k x[4*(l/16) + v][k] in xs[ci][v]
    f32x4_t xs[C];
    {
        const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
        for (int ci = 0; ci < C; ++ci) {
            xs[ci] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                xs[ci] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, xr[ci][s4]), __builtin_bit_cast(bf16x8_t, ones),
                    xs[ci], 0, 0, 0);
        }
    }
    __syncthreads();

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + TAB_BYTES);
    const bool split = args.S > 1;

    // The body is straight-line apart from uniform branches that skip the
    // decode of tiles past the sequence: every load is issued on every path, so
    // the in-flight ring survives the loop (no register copies, no early waits).
    for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = t0 + u;
            const int ci = u % C;
            const int i = t / C;   // block number in this workgroup's sequence
            if (ci == 0) {
                // start of block i: build the table of block i+1, then fetch the
                // table rows of block i+1+LR into the slot just used.
                const int q = (u / C + 1) % LR;
                tab_build((i + 1) & 1, lq0[q], lq1[q], llo[q]);
                lut_load(i + 1 + LR, lq0[q], lq1[q], llo[q]);
            }
            if (t < T) {
                // decode tile t
                const u32x4_t p = pb[u];
                const float a = bf16_to_f32(ab[u]);
                const float bt = bf16_to_f32(bbv[u]);
                const uint32_t slot4 = static_cast<uint32_t>((i & 1) * 128 + (lane & 31) * 4);
                f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    u32x4_t bw;
                    bw[0] = lds_word(smem, tab_addr(p[s4], slot4, 0));
                    bw[1] = lds_word(smem, tab_addr(p[s4], slot4, 1));
                    bw[2] = lds_word(smem, tab_addr(p[s4], slot4, 2));
                    bw[3] = lds_word(smem, tab_addr(p[s4], slot4, 3));
                    ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xr[ci][s4]), __builtin_bit_cast(bf16x8_t, bw),
                        ag, 0, 0, 0);
                }
#pragma unroll
                for (int v = 0; v < VC; ++v)
                    acc[v] = fmaf(a, ag[v], fmaf(bt, xs[ci][v], acc[v]));
            }
            issue(u, t + D);
            if (ci == C - 1) {
                // end of block i: partial sums of the 8 waves meet in LDS
                red[((i & 1) * GW + wave) * 64 + lane] = acc;
                acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                __syncthreads();
                if (wave == i % GW && i < nblk) {
                    f32x4_t tot = red[((i & 1) * GW) * 64 + lane];
#pragma unroll
                    for (int w = 1; w < GW; ++w) {
                        const f32x4_t o = red[((i & 1) * GW + w) * 64 + lane];
#pragma unroll
                        for (int v = 0; v < VC; ++v)
                            tot[v] += o[v];
                    }
                    const int b = r + i * args.Gp;
                    if (!split) {
                        const int n = b * TILE_ROWS + j;
#pragma unroll
                        for (int v = 0; v < VC; ++v) {
                            const int m = kq * 4 + v;
                            if (m < M && n < N)
                                args.y[static_cast<size_t>(m) * N + n] =
                                    static_cast<uint16_t>(f32_to_bf16(tot[v]));
                        }
                    } else {
                        float* pp =
                            args.part + ((static_cast<size_t>(s) * NB + b) * 64 + lane) * VC;
#pragma unroll
                        for (int v = 0; v < VC; ++v)
                            pp[v] = tot[v];
                    }
                }
            }
        }
    }

    if (!split)
        return;
    // ---- split K: the last workgroup to finish a block sums its S parts in order.
    for (int i = wave; i < nblk; i += GW) {
        const int b = r + i * args.Gp;
        __threadfence();
        uint32_t old = 0;
        if (lane == 0)
            old = atomicAdd(args.count + b, 1u);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != static_cast<uint32_t>(args.S - 1))
            continue;
        __threadfence();
        float tot[VC];
#pragma unroll
        for (int v = 0; v < VC; ++v)
            tot[v] = 0.f;
        for (int sp = 0; sp < args.S; ++sp) {
            const float* pp = args.part + ((static_cast<size_t>(sp) * NB + b) * 64 + lane) * VC;
#pragma unroll
            for (int v = 0; v < VC; ++v)
                tot[v] += __builtin_nontemporal_load(pp + v);
        }
        const int n = b * TILE_ROWS + j;
#pragma unroll
        for (int v = 0; v < VC; ++v) {
            const int m = kq * 4 + v;
            if (m < M && n < N)
                args.y[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16(tot[v]));
        }
        // leave this block's part of the workspace zero again, counter included
        for (int sp = 0; sp < args.S; ++sp) {
            float* pp = args.part + ((static_cast<size_t>(sp) * NB + b) * 64 + lane) * VC;
#pragma unroll
            for (int v = 0; v < VC; ++v)
                pp[v] = 0.f;
        }
        if (lane == 0)
            args.count[b] = 0u;
    }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool group_ok(int64_t K, int64_t g)
{
    return g > 0 && g % TILE_K == 0 && K >= 0 && K % g == 0;
}

int64_t row_blocks(int64_t N)
{
    return (N + TILE_ROWS - 1) / TILE_ROWS;
}

any4_status launched()
{
    return hipGetLastError() == hipSuccess ? ANY4_OK : ANY4_E_HIP;
}

// How a GEMM is split: C chunks per wave, S parts of K, Gp workgroups per part.
struct Plan {
    int C, S, Gp;
};

constexpr int PLAN_CUS = 256;   // the split is planned for a full MI355X

Plan plan_for(int64_t N, int64_t K)
{
    const int64_t Kc = K / TILE_K, NB = row_blocks(N);
    Plan best{4, 1, 1};
    double best_cost = 1e30;
    for (int C : {4, 2, 1}) {
        const int64_t S = (Kc + GW * C - 1) / (GW * C);
        int64_t Gp = PLAN_CUS / S;
        if (Gp < 1)
            Gp = 1;
        if (Gp > NB)
            Gp = NB;
        const int64_t rounds = (NB + Gp - 1) / Gp;
        // time of one workgroup: rounds x (C tiles + table build and barrier);
        // a split adds the partial-sum traffic and the final sum.
        const double cost = rounds * (C + 0.5) + (S > 1 ? 1.0 : 0.0);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = Plan{C, static_cast<int>(S), static_cast<int>(Gp)};
        }
    }
    return best;
}

size_t split_bytes(int64_t M, int64_t N, const Plan& p, size_t* count_off)
{
    if (p.S <= 1) {
        *count_off = 0;
        return 0;
    }
    const int64_t NB = row_blocks(N);
    const int64_t VC = M < 4 ? M : 4;
    const size_t part = static_cast<size_t>(p.S) * NB * 64 * VC * sizeof(float);
    *count_off = (part + 255) & ~static_cast<size_t>(255);
    return *count_off + static_cast<size_t>(NB) * sizeof(uint32_t);
}

template <int MT>
void launch_gemm(const Plan& p, const GemmArgs& a, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(p.S * p.Gp)), block(GT);
    switch (p.C) {
    case 4: hipLaunchKernelGGL((k_gemm<MT, 4, 8, 2>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<MT, 2, 8, 2>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((k_gemm<MT, 1, 8, 2>), grid, block, 0, stream, a); break;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* any4_status_string(any4_status s)
{
    switch (s) {
    case ANY4_OK: return "ANY4_OK: success";
    case ANY4_E_NULL: return "ANY4_E_NULL: a required pointer is NULL";
    case ANY4_E_SHAPE: return "ANY4_E_SHAPE: unsupported sizes (negative size, K not a multiple "
                              "of 128, g not a positive multiple of 128, K % g != 0, M > 16, "
                              "or buffers of 2 GiB or more)";
    case ANY4_E_ALIGN: return "ANY4_E_ALIGN: a base pointer is not aligned as required";
    case ANY4_E_WORKSPACE: return "ANY4_E_WORKSPACE: workspace too small";
    case ANY4_E_HIP: return "ANY4_E_HIP: the HIP runtime reported an error";
    }
    return "any4: unknown status";
}

size_t any4_packed_bytes(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % TILE_K != 0)
        return 0;
    return static_cast<size_t>(row_blocks(N)) * TILE_ROWS * static_cast<size_t>(K / 2);
}

any4_status any4_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream)
{
    if (N < 0 || K < 0 || K % TILE_K != 0)
        return ANY4_E_SHAPE;
    if (N == 0 || K == 0)
        return ANY4_OK;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(N) * K >= (static_cast<size_t>(1) << 40))
        return ANY4_E_SHAPE;
    if (!idx || !packed)
        return ANY4_E_NULL;
    if (!aligned(idx, 16) || !aligned(packed, 16))
        return ANY4_E_ALIGN;
    const uint32_t slots = static_cast<uint32_t>(any4_packed_bytes(N, K) / 16);
    const uint32_t blocks = (slots + PACK_THREADS - 1) / PACK_THREADS;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(PACK_THREADS), 0, stream, idx, packed,
                       static_cast<int>(N), static_cast<int>(K), slots);
    return launched();
}

any4_status any4_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream)
{
    if (N < 0 || !group_ok(K, g))
        return ANY4_E_SHAPE;
    if (N == 0 || K == 0)
        return ANY4_OK;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (!packed || !lut || !alpha || !beta || !w)
        return ANY4_E_NULL;
    if (!aligned(packed, 16) || !aligned(w, 16) || !aligned(lut, 2) || !aligned(alpha, 2) ||
        !aligned(beta, 2))
        return ANY4_E_ALIGN;
    const int64_t Kc = K / TILE_K;
    const int64_t blocks = row_blocks(N) * ((Kc + DQ_WAVES - 1) / DQ_WAVES);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_dequant, dim3(static_cast<unsigned>(blocks)), dim3(64 * DQ_WAVES), 0,
                       stream, packed, lut, alpha, beta, w, static_cast<int>(N),
                       static_cast<int>(K), static_cast<int>(g));
    return launched();
}

size_t any4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t g)
{
    if (M <= 0 || M > 16 || N <= 0 || K <= 0 || !group_ok(K, g))
        return 0;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31))
        return 0;
    size_t off = 0;
    return split_bytes(M, N, plan_for(N, K), &off);
}

any4_status any4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    if (M < 0 || M > 16 || N < 0 || !group_ok(K, g))
        return ANY4_E_SHAPE;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(M) * K * 2 >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (M == 0 || N == 0)
        return ANY4_OK;
    if (!y || (K > 0 && (!x || !packed || !lut || !alpha || !beta)))
        return ANY4_E_NULL;
    if (!aligned(y, 2) || (K > 0 && (!aligned(x, 16) || !aligned(packed, 16) ||
                                     !aligned(lut, 16) || !aligned(alpha, 2) ||
                                     !aligned(beta, 2))))
        return ANY4_E_ALIGN;
    (void)hipGetLastError();
    if (K == 0) {
        const size_t n = static_cast<size_t>(M) * N;
        hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                           stream, y, n);
        return launched();
    }
    const Plan p = plan_for(N, K);
    size_t count_off = 0;
    const size_t need = split_bytes(M, N, p, &count_off);
    if (workspace_bytes < need)
        return ANY4_E_WORKSPACE;
    if (need > 0 && (!workspace || !aligned(workspace, 256)))
        return workspace ? ANY4_E_ALIGN : ANY4_E_NULL;
    GemmArgs a;
    a.x = x;
    a.packed = packed;
    a.lut = lut;
    a.alpha = alpha;
    a.beta = beta;
    a.y = y;
    a.part = need ? static_cast<float*>(workspace) : nullptr;
    a.count = need ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + count_off)
                   : nullptr;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.g = static_cast<int>(g);
    a.S = p.S;
    a.Gp = p.Gp;
    if (M == 1)
        launch_gemm<1>(p, a, stream);
    else if (M == 2)
        launch_gemm<2>(p, a, stream);
    else if (M <= 4)
        launch_gemm<4>(p, a, stream);
    else if (M <= 8)
        launch_gemm<8>(p, a, stream);
    else
        launch_gemm<16>(p, a, stream);
    return launched();
}

}  // extern "C"
