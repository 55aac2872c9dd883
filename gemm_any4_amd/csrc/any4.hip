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

// The same with the non-temporal hint, for data read exactly once (weights).
__device__ __forceinline__ u32x4_t load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
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

// Two kernels compute y = x * W^T; both work on 16-row blocks of W, with the
// 8 waves of a workgroup splitting the block's K and meeting in LDS.
//
//   k_gemm_res  (K <= 4096) persistent: about one workgroup per CU walks row
//               blocks r, r+G, r+2G, ...; wave w always decodes the same 4
//               chunks of 128 k, so their x operands are loaded once, into
//               VGPRs, and reused for every block.
//   k_gemm_str  (any K) one workgroup per row block; a wave decodes K/8 of
//               the block and loads the x operand of each chunk with the
//               chunk's tile.
//
// Decode.  A packed byte (two indices) selects one dword of a pair table in
// LDS: entry (hi << 4 | lo) holds (LUT[lo], LUT[hi]) as two bf16, which is
// exactly one dword of an MFMA B operand.  The table of a row block has 32
// slots per entry (slot = lane % 32, row = slot % 16); a wave64 LDS read is
// served as two halves of 32 lanes, so every lane reads its own bank: no
// conflicts.  Entry e of table buffer q sits at byte e*256 + q*128, so the
// read address is one v_perm of the packed dword.
//
// Scale and offset.  Per 128-k chunk a lane accumulates sum_k x*LUT[idx] with
// four MFMAs, then adds alpha times that sum, plus beta times sum_k x.
//
// Staging.  The table rows (16 x 32 B) and the block's alpha and beta
// (16 x K/g bf16 each, contiguous in [N][K/g]) are fetched with coalesced
// 16-byte loads and written to LDS, alpha and beta interleaved as
// (alpha | beta << 16) dwords, so a lane reads both with one ds_read_b32.
//
// Memory.  Each wave keeps the next D tiles of its sequence in flight in a
// register ring.  Every load is a bounds-checked buffer load whose offset is
// pushed out of range where there is nothing to read (past the wave's work,
// x rows m >= M), so no branch guards a load and no traffic is made.  The
// loop bodies are straight-line apart from uniform branches that skip the
// decode of tiles past the sequence, so the ring survives the loop.
constexpr int GW = 8;                   // waves per workgroup
constexpr int GT = 64 * GW;
constexpr int TAB_BYTES = 256 * 256;    // 256 entries x 2 buffers x 32 slots x 4 B
constexpr int RES_MAX_K = 4096;         // k_gemm_res: K covered by one workgroup
constexpr int STR_MAX_G = 512;          // k_gemm_str: K/g up to 512 (two staging rounds)

struct GemmArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* lut;
    const uint16_t* alpha;
    const uint16_t* beta;
    uint16_t* y;
    int M, N, K, g;
};

// Byte address of table entry `byte j of d` in the lane's slot: (d.byte[j] << 8) | slot4.
__device__ __forceinline__ uint32_t tab_addr(uint32_t d, uint32_t slot4, int j)
{
    return __builtin_amdgcn_perm(d, slot4, 0x0C0C0000u | ((4u + j) << 8));
}

template <typename T>
__device__ __forceinline__ T& lds_at(uint8_t* smem, uint32_t byte_addr)
{
    return *reinterpret_cast<T*>(smem + byte_addr);
}

// Build table buffer `buf` of one row block from its 16 LUT rows, staged in
// LDS at `lut_off` as [16 rows][16] bf16.  Thread t of the W*64 writes slot
// t % 32 (row (t % 32) % 16) of the entries lo + 16*hi, lo = (t / 32) % 16,
// for its share of the 16 hi.
template <int W>
__device__ __forceinline__ void build_table(uint8_t* smem, uint32_t lut_off, int buf, int tid)
{
    constexpr int HPT = 128 / W;   // hi values per thread
    const int st = tid & 31;
    const int lo = (tid >> 5) & 15;
    const int h0 = (tid >> 9) * HPT;
    const uint32_t row = lut_off + (st & 15) * 32;
    const u32x4_t q0 = lds_at<u32x4_t>(smem, row);
    const u32x4_t q1 = lds_at<u32x4_t>(smem, row + 16);
    const uint32_t ll = lds_at<uint16_t>(smem, row + 2 * lo);
    const uint32_t Lw[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
    uint32_t* tw = reinterpret_cast<uint32_t*>(smem) + lo * 64 + buf * 32 + st;
    if constexpr (HPT == 16) {
#pragma unroll
        for (int hi = 0; hi < 16; ++hi)
            tw[hi * 16 * 64] =
                __builtin_amdgcn_perm(Lw[hi >> 1], ll, (hi & 1) ? 0x07060100u : 0x05040100u);
    } else {
#pragma unroll
        for (int hh = 0; hh < HPT; ++hh) {
            const int hi = h0 + hh;
            uint32_t v = Lw[0];
#pragma unroll
            for (int q = 1; q < 8; ++q)
                if (hi >> 1 == q)
                    v = Lw[q];
            tw[hi * 16 * 64] = __builtin_amdgcn_perm(v, ll, (hi & 1) ? 0x07060100u : 0x05040100u);
        }
    }
}

// Interleave 8 alpha and 8 beta values (elements 8q .. 8q+7 of the block's
// [16][G] arrays) into (alpha | beta << 16) dwords stored as [group][row]:
// the 16 rows of a group are 16 consecutive dwords, so the 16 rows' lanes
// read 16 different banks.
__device__ __forceinline__ void store_pairs(uint8_t* smem, uint32_t base, int q, int G,
                                            const u32x4_t& qa, const u32x4_t& qb)
{
    int row = (8 * q) / G;
    int grp = 8 * q - row * G;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        lds_at<uint32_t>(smem, base + (grp * 16 + row) * 4) =
            __builtin_amdgcn_perm(qb[i >> 1], qa[i >> 1], sel);
        if (++grp == G) {
            grp = 0;
            ++row;
        }
    }
}

// sum_k x*LUT[idx] over one tile: four MFMAs, B operands looked up in the
// table through `slot4` (buffer and slot of this lane).
__device__ __forceinline__ f32x4_t tile_dot(const uint8_t* smem, uint32_t slot4, const u32x4_t& p,
                                            const u32x4_t (&xa)[4])
{
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        u32x4_t bw;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            bw[jb] = *reinterpret_cast<const uint32_t*>(smem + tab_addr(p[s4], slot4, jb));
        ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[s4]),
                                                     __builtin_bit_cast(bf16x8_t, bw), ag, 0, 0,
                                                     0);
    }
    return ag;
}

// The 8 waves' partial sums of one block, left by each wave in red[wave][lane],
// summed in wave order; lane l holds y[4*(l/16) + v][n0 + l%16].
template <int MT, int W>
__device__ __forceinline__ void store_block(const f32x4_t* red, uint16_t* y, int lane, int M,
                                            int N, int n0)
{
    constexpr int VC = MT < 4 ? MT : 4;
    f32x4_t tot = red[lane];
#pragma unroll
    for (int w = 1; w < W; ++w) {
        const f32x4_t o = red[w * 64 + lane];
#pragma unroll
        for (int v = 0; v < VC; ++v)
            tot[v] += o[v];
    }
    const int n = n0 + (lane & 15);
#pragma unroll
    for (int v = 0; v < VC; ++v) {
        const int m = (lane >> 4) * 4 + v;
        if (m < M && n < N)
            y[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16(tot[v]));
    }
}

// ---- k_gemm_res: persistent, x resident in VGPRs (K <= 4096) -------------
//
// W waves of C chunks each cover K <= W*C*128 = 4096.  LDS: [0, 64K) tables
// (2 buffers), red[2][W][64] f32x4, alpha/beta pairs [2][G <= 32][16] dwords,
// LUT rows [2][16][16] bf16, then (M <= XRMAX) x staging [W][M][C*256 B].
// Pipeline at the start of block i (all waves), parity P = i & 1 known at
// compile time (the loop body covers two blocks):
//   build table (i+1)&1 from LUT rows (i+1)&1          (staged at block i-1)
//   pairs (i+1)&1   <- alpha/beta registers P^1         (loaded at block i-1)
//   LUT rows i&1    <- LUT registers P (block i+2)      (loaded at block i-2)
//   load alpha/beta of block i+3 into registers P^1, LUT of block i+4 into P
// and the barrier at the end of block i publishes what block i+1 reads.
template <int W, int C>
struct ResCfg {
    static constexpr int T = 64 * W;                  // threads
    static constexpr int D = 2 * C;                   // ring: two blocks of tiles
    static constexpr int RED = TAB_BYTES;
    static constexpr int AB = RED + 2 * W * 64 * 16;
    static constexpr int AB_BYTES = 16 * (RES_MAX_K / TILE_K) * 4;   // [G <= 32][16] dwords
    static constexpr int LUT = AB + 2 * AB_BYTES;
    static constexpr int XS = LUT + 2 * 512;
    // rows of x that go through LDS on their way to the MFMA operands: a wave
    // fetches each row of its C*128 k with one full-width load, instead of
    // 4C loads in which only the M lanes of the operand layout are live
    static constexpr int XRMAX = W <= 8 ? 8 : 4;
    template <int MT>
    static constexpr int x_rows() { return MT <= XRMAX ? MT : 0; }
    template <int MT>
    static constexpr int lds() { return XS + W * x_rows<MT>() * C * 256; }
};

template <int MT, int W, int C>
__global__ __launch_bounds__(64 * W) void k_gemm_res(const GemmArgs args)
{
    using Cfg = ResCfg<W, C>;
    constexpr int D = Cfg::D;
    constexpr int VC = MT < 4 ? MT : 4;
    constexpr int XR = Cfg::template x_rows<MT>();
    static_assert(W * C * TILE_K == RES_MAX_K, "one part covers K <= 4096");
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::template lds<MT>()];

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;      // tile row of this lane (B operand), x row m (A operand)
    const int kq = lane >> 4;     // 32-k quarter of a chunk
    const int Kc = K / TILE_K;
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = K / g;
    const int Gs = gridDim.x;
    const int r = blockIdx.x;
    const int nblk = r < NB ? (NB - 1 - r) / Gs + 1 : 0;
    const int T = nblk * C;               // tiles in this wave's sequence
    const int cbase = wave * C;

    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TILE_BYTES);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, static_cast<uint32_t>(N) * 32);
    // alpha/beta are staged with 16-byte loads: the range is rounded up to 16 B
    // (the 16-byte granule holding a valid byte never leaves that byte's page
    // when the base is 16-byte aligned); the extra values only reach rows >= N.
    const uint32_t ab_range = (static_cast<uint32_t>(N) * G * 2 + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, ab_range);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, ab_range);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // staging loads of block i: thread t < 32 fetches 16 B of the LUT rows,
    // thread t < 2G fetches 16 B of alpha and of beta.  Offsets = a per-lane
    // part (OOR for lanes with nothing to fetch) plus a uniform block part;
    // blocks past the last one lie past the buffers, so no per-lane select
    // (which the compiler may turn into branches) is needed.
    const uint32_t ab_bytes = static_cast<uint32_t>(G) * 32;   // 16 rows x G x 2 B
    const uint32_t lut_lane = tid < 32 ? static_cast<uint32_t>(tid) * 16 : OOR;
    const uint32_t ab_lane = static_cast<uint32_t>(tid) * 16 < ab_bytes ? tid * 16 : OOR;
    auto lut_load = [&](int i) {
        return load16(rl, lut_lane + static_cast<uint32_t>(r + i * Gs) * 512);
    };
    auto ab_load = [&](int i, u32x4_t& qa, u32x4_t& qb) {
        const uint32_t off = ab_lane + static_cast<uint32_t>(r + i * Gs) * ab_bytes;
        qa = load16(ra, off);
        qb = load16(rb, off);
    };
    auto lut_stage = [&](int buf, const u32x4_t& q) {
        if (tid < 32)
            lds_at<u32x4_t>(smem, Cfg::LUT + buf * 512 + tid * 16) = q;
    };
    auto ab_stage = [&](int buf, const u32x4_t& qa, const u32x4_t& qb) {
        if (static_cast<uint32_t>(tid) * 16 < ab_bytes)
            store_pairs(smem, Cfg::AB + buf * Cfg::AB_BYTES, tid, G, qa, qb);
    };

    // ---- tile ring (streamed once: non-temporal loads)
    u32x4_t pb[D];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * 16;
    auto issue = [&](int u, int t) {
        const int i = t / C;
        const int c = cbase + t % C;
        const bool live = t < T && c < Kc;
        const int b = r + i * Gs;
        pb[u] = load16_nt(rp, live ? static_cast<uint32_t>(b * Kc + c) * TILE_BYTES + tile_lane
                                   : OOR);
    };

    // ---- prologue.  The loads of the staging registers go out before the
    // ring, as they do in the loop, so that the waits the compiler derives for
    // the loop (from both of its entries) leave the ring in flight.
    u32x4_t l0 = lut_load(0), l1 = lut_load(1), a0, b0;
    ab_load(0, a0, b0);
    u32x4_t lq[2], aq[2], bq[2];
    lq[0] = lut_load(2);
    lq[1] = lut_load(3);
    ab_load(1, aq[1], bq[1]);
    ab_load(2, aq[0], bq[0]);
    u32x4_t xr[C][4];
    u32x4_t xw[XR > 0 ? XR : 1];
    if constexpr (XR > 0) {
        // row m of x over this wave's C*128 k: lane l < 16C holds k = 8l .. 8l+7
        const int k0 = cbase * TILE_K + lane * 8;
        const uint32_t xk = (lane < 16 * C && k0 < K) ? static_cast<uint32_t>(k0) * 2 : OOR;
#pragma unroll
        for (int m = 0; m < XR; ++m)
            xw[m] = load16(rx, m < M ? xk + static_cast<uint32_t>(m * K) * 2 : OOR);
    } else {
        const uint32_t x_lane = j < M ? static_cast<uint32_t>(j * K + kq * 32) * 2 : OOR;
#pragma unroll
        for (int ci = 0; ci < C; ++ci) {
            const int c = cbase + ci;
            const uint32_t xc = c < Kc ? static_cast<uint32_t>(c) * TILE_K * 2 : OOR;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                xr[ci][s4] = load16(rx, (x_lane | (xc & OOR)) + (xc & ~OOR) + s4 * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
        issue(u, u);
    if constexpr (XR > 0) {
        // through this wave's own LDS rows into the operand layout: lane
        // (j, kq) takes row j, k = 128 ci + 32 kq + 8 s4 .. +8 (zero for j >= M)
        constexpr int ROW = C * 256;
        const uint32_t xs_base = Cfg::XS + wave * XR * ROW;
        if (lane < 16 * C) {
#pragma unroll
            for (int m = 0; m < XR; ++m)
                lds_at<u32x4_t>(smem, xs_base + m * ROW + lane * 16) = xw[m];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int ci = 0; ci < C; ++ci)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                xr[ci][s4] = u32x4_t{0u, 0u, 0u, 0u};
        if (j < M) {
            const uint32_t rb0 = xs_base + j * ROW + kq * 64;
#pragma unroll
            for (int ci = 0; ci < C; ++ci)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    xr[ci][s4] = lds_at<u32x4_t>(smem, rb0 + ci * 256 + s4 * 16);
        }
    }
    lut_stage(0, l0);
    lut_stage(1, l1);
    ab_stage(0, a0, b0);
    __syncthreads();
    build_table<W>(smem, Cfg::LUT, 0, tid);

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
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + Cfg::RED);
    const uint32_t slot_lane = static_cast<uint32_t>(lane & 31) * 4;
    int gi_c[C];
#pragma unroll
    for (int ci = 0; ci < C; ++ci)
        gi_c[ci] = ((cbase + ci) * TILE_K) / g;

    for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = t0 + u;
            const int ci = u % C;
            const int P = (u / C) & 1;  // parity of block i
            const int i = t / C;
            if (ci == 0) {
                build_table<W>(smem, Cfg::LUT + ((i + 1) & 1) * 512, (i + 1) & 1, tid);
                ab_stage(P ^ 1, aq[P ^ 1], bq[P ^ 1]);
                lut_stage(P, lq[P]);
                ab_load(i + 3, aq[P ^ 1], bq[P ^ 1]);
                lq[P] = lut_load(i + 4);
            }
            {
                // no branch around the decode, so the scheduler can overlap
                // tiles; a tile past the sequence gets alpha = beta = 0
                const uint32_t pr = t < T ? lds_at<uint32_t>(smem, Cfg::AB + P * Cfg::AB_BYTES +
                                                                       (gi_c[ci] * 16 + j) * 4)
                                          : 0u;
                const f32x4_t ag = tile_dot(smem, P * 128 + slot_lane, pb[u], xr[ci]);
                const float a = bf16_to_f32(pr & 0xFFFFu);
                const float bt = bf16_to_f32(pr >> 16);
#pragma unroll
                for (int v = 0; v < VC; ++v)
                    acc[v] = fmaf(a, ag[v], fmaf(bt, xs[ci][v], acc[v]));
            }
            issue(u, t + D);
            if (ci == C - 1) {
                red[(P * W + wave) * 64 + lane] = acc;
                acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                __syncthreads();
                if (wave == i % W && i < nblk)
                    store_block<MT, W>(red + P * W * 64, args.y, lane, M, N,
                                       (r + i * Gs) * TILE_ROWS);
            }
        }
    }
}

// ---- k_gemm_str: one row block per workgroup, x loaded per tile ----------
//
// LDS: [0, 64K) table (buffer 0 used), red[8][64] f32x4 (8 KB), alpha/beta
// pairs [16][K/g] dwords (<= 32 KB), LUT rows [16][16] bf16.
constexpr int STR_D = 8;
constexpr int STR_RED = TAB_BYTES;
constexpr int STR_AB = STR_RED + GW * 64 * 16;
constexpr int STR_LUT = STR_AB + 16 * STR_MAX_G * 4;
constexpr int STR_LDS = STR_LUT + 512;

template <int MT>
__global__ __launch_bounds__(GT) void k_gemm_str(const GemmArgs args)
{
    constexpr int D = STR_D;
    constexpr int VC = MT < 4 ? MT : 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[STR_LDS];

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int kq = lane >> 4;
    const int Kc = K / TILE_K;
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = K / g;
    const int b = blockIdx.x;
    const int CB = (Kc + GW - 1) / GW;   // tiles per wave
    const int c0 = wave * CB;

    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TILE_BYTES);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, static_cast<uint32_t>(N) * 32);
    // alpha/beta are staged with 16-byte loads: the range is rounded up to 16 B
    // (the 16-byte granule holding a valid byte never leaves that byte's page
    // when the base is 16-byte aligned); the extra values only reach rows >= N.
    const uint32_t ab_range = (static_cast<uint32_t>(N) * G * 2 + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, ab_range);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, ab_range);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // staging loads first, so that waiting for them leaves the ring in flight
    const uint32_t ab_bytes = static_cast<uint32_t>(G) * 32;
    const u32x4_t lq =
        load16(rl, (tid < 32 ? static_cast<uint32_t>(tid) * 16 : OOR) + static_cast<uint32_t>(b) * 512);
    u32x4_t aq[2], bq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t o = static_cast<uint32_t>(tid + h * GT) * 16;
        const uint32_t off = (o < ab_bytes ? o : OOR) + static_cast<uint32_t>(b) * ab_bytes;
        aq[h] = load16(ra, off);
        bq[h] = load16(rb, off);
    }

    u32x4_t pb[D];
    u32x4_t px[D][4];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * 16;
    // x rows m >= M: a per-lane out-of-range base; dead tiles: a uniform one
    const uint32_t x_lane = j < M ? static_cast<uint32_t>(j * K + kq * 32) * 2 : OOR;
    auto issue = [&](int u, int t) {
        const int c = c0 + t;
        const bool live = t < CB && c < Kc;
        pb[u] = load16(rp, live ? static_cast<uint32_t>(b * Kc + c) * TILE_BYTES + tile_lane : OOR);
        const uint32_t xc = live ? static_cast<uint32_t>(c) * TILE_K * 2 : OOR;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
            px[u][s4] = load16(rx, (x_lane | (xc & OOR)) + (xc & ~OOR) + s4 * 16);
    };
#pragma unroll
    for (int u = 0; u < D; ++u)
        issue(u, u);

    if (tid < 32)
        lds_at<u32x4_t>(smem, STR_LUT + tid * 16) = lq;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (static_cast<uint32_t>(tid + h * GT) * 16 < ab_bytes)
            store_pairs(smem, STR_AB, tid + h * GT, G, aq[h], bq[h]);
    __syncthreads();
    build_table<GW>(smem, STR_LUT, 0, tid);
    __syncthreads();

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t slot4 = static_cast<uint32_t>(lane & 31) * 4;
    for (int t0 = 0; t0 < CB; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int t = t0 + u;
            const int c = c0 + t;
            if (t < CB && c < Kc) {
                const uint32_t pr =
                    lds_at<uint32_t>(smem, STR_AB + (((c * TILE_K) / g) * 16 + j) * 4);
                const float a = bf16_to_f32(pr & 0xFFFFu);
                const uint32_t b2 = (pr & 0xFFFF0000u) | (pr >> 16);
                const u32x4_t bv = {b2, b2, b2, b2};
                const f32x4_t ag = tile_dot(smem, slot4, pb[u], px[u]);
#pragma unroll
                for (int v = 0; v < VC; ++v)
                    acc[v] = fmaf(a, ag[v], acc[v]);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, px[u][s4]), __builtin_bit_cast(bf16x8_t, bv),
                        acc, 0, 0, 0);
            }
            issue(u, t + D);
        }
    }

    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + STR_RED);
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0)
        store_block<MT, GW>(red, args.y, lane, M, N, b * TILE_ROWS);
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

constexpr int RES_GRID = 256;   // k_gemm_res: one workgroup per CU of an MI355X
#ifndef ANY4_RES_WAVES
#define ANY4_RES_WAVES 8
#endif
constexpr int RES_W = ANY4_RES_WAVES;
constexpr int RES_CW = RES_MAX_K / TILE_K / RES_W;

template <int MT>
void launch_gemm(const GemmArgs& a, hipStream_t stream)
{
    const int64_t NB = row_blocks(a.N);
    if (a.K <= RES_MAX_K) {
        const int grid = static_cast<int>(NB < RES_GRID ? NB : RES_GRID);
        hipLaunchKernelGGL((k_gemm_res<MT, RES_W, RES_CW>), dim3(grid), dim3(64 * RES_W), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL(k_gemm_str<MT>, dim3(static_cast<unsigned>(NB)), dim3(GT), 0, stream,
                           a);
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
                              "of 128, g not a positive multiple of 128, K % g != 0, K/g > 512, "
                              "M > 16, or buffers of 2 GiB or more)";
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
    (void)M;
    (void)N;
    (void)K;
    (void)g;
    return 0;   // neither kernel needs device scratch
}

any4_status any4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (M < 0 || M > 16 || N < 0 || !group_ok(K, g) || K / (g > 0 ? g : 1) > STR_MAX_G)
        return ANY4_E_SHAPE;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(M) * K * 2 >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(N) * 32 >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (M == 0 || N == 0)
        return ANY4_OK;
    if (!y || (K > 0 && (!x || !packed || !lut || !alpha || !beta)))
        return ANY4_E_NULL;
    if (!aligned(y, 2) || (K > 0 && (!aligned(x, 16) || !aligned(packed, 16) ||
                                     !aligned(lut, 16) || !aligned(alpha, 16) ||
                                     !aligned(beta, 16))))
        return ANY4_E_ALIGN;
    (void)hipGetLastError();
    if (K == 0) {
        const size_t n = static_cast<size_t>(M) * N;
        hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                           stream, y, n);
        return launched();
    }
    GemmArgs a;
    a.x = x;
    a.packed = packed;
    a.lut = lut;
    a.alpha = alpha;
    a.beta = beta;
    a.y = y;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.g = static_cast<int>(g);
    if (M == 1)
        launch_gemm<1>(a, stream);
    else if (M == 2)
        launch_gemm<2>(a, stream);
    else if (M <= 4)
        launch_gemm<4>(a, stream);
    else if (M <= 8)
        launch_gemm<8>(a, stream);
    else
        launch_gemm<16>(a, stream);
    return launched();
}

}  // extern "C"
