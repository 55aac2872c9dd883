// libany4 -- any4 dequantize-GEMM for MI355X (gfx950, CDNA4).
//
// What is computed (the 10100.com any4 explainer): each weight is a 4-bit index
// into its row's 16-entry bf16 table (section 二), each contiguous group of g
// weights of a row has a scale alpha and an offset beta (step 1, "分组缩放"), so
// w = alpha * LUT_row[idx] + beta; the matmul y = x * W^T runs at decode batch
// sizes 1..16 (section 三).  The C ABI is declared in include/any4.h.
//
// Kernels
//   k_pack     nibble packing, 32 index bytes -> 16 packed bytes per thread.
//   k_dequant  w = bf16(fma(alpha, LUT[idx], beta)), 16 weights per thread.
//   k_gemm     y = x * W^T on the bf16 MFMA units:
//     * A 16-row tile of W is the B operand of v_mfma_f32_16x16x32_bf16, x is
//       the A operand (rows m >= M are zero), so one MFMA covers 16 weight rows
//       x 32 k for every m of the batch.
//     * Lookup: each packed byte (two indices) selects one dword of a per-lane
//       LDS table holding the bf16 pair (LUT[lo], LUT[hi]), which is exactly one
//       dword of the MFMA operand.  The table has 256 entries x 64 slots, one
//       slot per lane, laid out entry-major, so a lane always reads bank
//       (lane mod 64): the gather is free of bank conflicts.  The byte address
//       entry*256 + lane*4 is one v_perm_b32 of the packed dword.
//     * Scale and offset stay out of the per-weight work: a group contributes
//       alpha * (sum_k x*LUT[idx]) + beta * (sum_k x); the first sum is an MFMA
//       chain, alpha is one FMA per accumulator, and the beta term is an MFMA
//       against a constant operand filled with beta.
//     * The waves of a workgroup share one tile and split its K; their partial
//       sums meet in LDS in a fixed order (deterministic), then are rounded to
//       bf16 and stored.
#include <hip/hip_runtime.h>

#include "any4.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32, round to
// nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
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

__global__ __launch_bounds__(PACK_THREADS) void k_pack(const uint8_t* __restrict__ idx,
                                                       uint8_t* __restrict__ packed,
                                                       size_t nout)
{
    const size_t o = (static_cast<size_t>(blockIdx.x) * PACK_THREADS + threadIdx.x) * 16;
    if (o + 16 <= nout) {
        const uint4* src = reinterpret_cast<const uint4*>(idx + 2 * o);
        const uint4 a = src[0], b = src[1];
        uint4 r;
        r.x = pack8(a.x, a.y);
        r.y = pack8(a.z, a.w);
        r.z = pack8(b.x, b.y);
        r.w = pack8(b.z, b.w);
        *reinterpret_cast<uint4*>(packed + o) = r;
    } else if (o < nout) {
        for (size_t j = o; j < nout; ++j)
            packed[j] = static_cast<uint8_t>((idx[2 * j] & 15u) | ((idx[2 * j + 1] & 15u) << 4));
    }
}

// ---------------------------------------------------------------------------
// dequant
// ---------------------------------------------------------------------------
constexpr int DQ_THREADS = 256;
constexpr int DQ_PER_THREAD = 16;                         // weights per thread
constexpr int DQ_PER_BLOCK = DQ_THREADS * DQ_PER_THREAD;  // 4096
constexpr int DQ_MAX_ROWS = DQ_PER_BLOCK / 128 + 1;       // K >= 128

__global__ __launch_bounds__(DQ_THREADS) void k_dequant(const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ lut,
                                                        const uint16_t* __restrict__ alpha,
                                                        const uint16_t* __restrict__ beta,
                                                        uint16_t* __restrict__ w, int64_t K,
                                                        int64_t g, size_t units)
{
    __shared__ float slut[DQ_MAX_ROWS * 16];
    const size_t u0 = static_cast<size_t>(blockIdx.x) * DQ_THREADS;
    const size_t ulast = min(u0 + DQ_THREADS, units) - 1;
    const int64_t n_first = static_cast<int64_t>(u0 * DQ_PER_THREAD / K);
    const int64_t n_last = static_cast<int64_t>(ulast * DQ_PER_THREAD / K);
    const int nrows = static_cast<int>(n_last - n_first + 1);
    for (int t = threadIdx.x; t < nrows * 16; t += DQ_THREADS)
        slut[t] = bf16_to_f32(lut[n_first * 16 + t]);
    __syncthreads();

    const size_t u = u0 + threadIdx.x;
    if (u >= units)
        return;
    const size_t e0 = u * DQ_PER_THREAD;                 // flat weight index
    const int64_t n = static_cast<int64_t>(e0 / K);
    const int64_t k0 = static_cast<int64_t>(e0 % K);
    const int64_t G = K / g;
    const float a = bf16_to_f32(alpha[n * G + k0 / g]);
    const float b = bf16_to_f32(beta[n * G + k0 / g]);
    const float* L = slut + (n - n_first) * 16;
    const uint2 p = *reinterpret_cast<const uint2*>(packed + e0 / 2);
    const uint32_t pw[2] = {p.x, p.y};
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t byte = (pw[q >> 2] >> (8 * (q & 3))) & 0xFFu;
        const float lo = fmaf(a, L[byte & 15u], b);
        const float hi = fmaf(a, L[byte >> 4], b);
        out[q] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(w + e0);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// ---------------------------------------------------------------------------
// gemm
// ---------------------------------------------------------------------------
constexpr int GEMM_WAVES = 8;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int TILE_N = 16;       // weight rows per tile (MFMA N)
constexpr int CHUNK_K = 128;     // k per chunk: a lane reads 16 packed bytes = 32 k
constexpr int TAB_SLOTS = 64;    // one table copy per lane
constexpr int TAB_WORDS = 256 * TAB_SLOTS;

// Byte address of table entry `byte j of d` in this lane's slot:
// (d.byte[j] << 8) | (lane * 4).
__device__ __forceinline__ uint32_t tab_addr(uint32_t d, uint32_t slot4, int j)
{
    return __builtin_amdgcn_perm(d, slot4, 0x0C0C0000u | ((4u + j) << 8));
}

__device__ __forceinline__ uint32_t tab_read(const uint32_t* tab, uint32_t byte_addr)
{
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(tab) + byte_addr);
}

template <int MT>
__global__ __launch_bounds__(GEMM_THREADS) void k_gemm(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ packed,
                                                       const uint16_t* __restrict__ lut,
                                                       const uint16_t* __restrict__ alpha,
                                                       const uint16_t* __restrict__ beta,
                                                       uint16_t* __restrict__ y, int M, int N,
                                                       int K, int g)
{
    __shared__ uint32_t tab[TAB_WORDS];   // 64 KB pair table, then the reduction buffer
    constexpr int VC = MT < 4 ? MT : 4;   // accumulator rows that can hold a real m

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;              // weight row in the tile, and x row m
    const int kq = lane >> 4;             // which 32-k quarter of a chunk
    const int nchunks = K / CHUNK_K;
    const int G = K / g;
    const int cpg = g / CHUNK_K;
    const int c_begin = nchunks * wave / GEMM_WAVES;
    const int c_end = nchunks * (wave + 1) / GEMM_WAVES;
    const int ntiles = (N + TILE_N - 1) / TILE_N;
    const bool has_x = j < M;
    const uint32_t slot4 = static_cast<uint32_t>(lane) * 4u;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int n0 = tile * TILE_N;
        const int nr = min(n0 + j, N - 1);   // rows past N read row N-1, never stored

        __syncthreads();   // the previous tile's reduction reads are done
        {
            const uint4* lp = reinterpret_cast<const uint4*>(lut + static_cast<size_t>(nr) * 16);
            const uint4 q0 = lp[0], q1 = lp[1];
            const uint32_t Lw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            constexpr int HPW = 16 / GEMM_WAVES;
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
                const int hi = wave * HPW + h;
                const uint32_t Lhi = lut[static_cast<size_t>(nr) * 16 + hi];
#pragma unroll
                for (int lo = 0; lo < 16; ++lo)
                    tab[(hi * 16 + lo) * TAB_SLOTS + lane] = __builtin_amdgcn_perm(
                        Lhi, Lw[lo >> 1], (lo & 1) ? 0x05040302u : 0x05040100u);
            }
        }
        __syncthreads();

        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const uint8_t* prow = packed + static_cast<size_t>(nr) * (K / 2) + kq * 16;
        const uint16_t* xr = x + static_cast<size_t>(has_x ? j : 0) * K + kq * 32;
        const uint16_t* arow = alpha + static_cast<size_t>(nr) * G;
        const uint16_t* brow = beta + static_cast<size_t>(nr) * G;
        for (int c = c_begin; c < c_end; ++c) {
            const uint4 p = *reinterpret_cast<const uint4*>(prow + static_cast<size_t>(c) * 64);
            u32x4_t xa[4];
            if (has_x) {
                const uint4* xp = reinterpret_cast<const uint4*>(xr + static_cast<size_t>(c) * CHUNK_K);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 v = xp[s];
                    xa[s] = u32x4_t{v.x, v.y, v.z, v.w};
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xa[s] = u32x4_t{0u, 0u, 0u, 0u};
            }
            const uint32_t pd[4] = {p.x, p.y, p.z, p.w};
            f32x4_t accg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4_t b;
                b[0] = tab_read(tab, tab_addr(pd[s], slot4, 0));
                b[1] = tab_read(tab, tab_addr(pd[s], slot4, 1));
                b[2] = tab_read(tab, tab_addr(pd[s], slot4, 2));
                b[3] = tab_read(tab, tab_addr(pd[s], slot4, 3));
                accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, xa[s]), __builtin_bit_cast(bf16x8_t, b), accg,
                    0, 0, 0);
            }
            const int grp = c / cpg;
            const float a = bf16_to_f32(arow[grp]);
            const uint32_t bb = brow[grp];
            const uint32_t b2 = bb | (bb << 16);
            const u32x4_t bv = {b2, b2, b2, b2};
#pragma unroll
            for (int v = 0; v < VC; ++v)
                acc[v] = fmaf(a, accg[v], acc[v]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, xa[s]), __builtin_bit_cast(bf16x8_t, bv), acc, 0,
                    0, 0);
        }

        __syncthreads();   // every wave is done with the table
        f32x4_t* red = reinterpret_cast<f32x4_t*>(tab);
        red[wave * 64 + lane] = acc;
        __syncthreads();
        for (int t = threadIdx.x; t < TILE_N * MT; t += GEMM_THREADS) {
            const int m = t >> 4, jj = t & 15;
            const int l = ((m >> 2) << 4) | jj, v = m & 3;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < GEMM_WAVES; ++w)
                s += red[w * 64 + l][v];
            if (m < M && n0 + jj < N)
                y[static_cast<size_t>(m) * N + n0 + jj] = static_cast<uint16_t>(f32_to_bf16(s));
        }
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
    return g > 0 && g % 128 == 0 && K >= 0 && K % g == 0;
}

constexpr int MAX_DEVICES = 64;
int g_cu_count[MAX_DEVICES];   // 0 = not queried yet

any4_status cu_count(int* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return ANY4_E_HIP;
    if (dev >= 0 && dev < MAX_DEVICES && g_cu_count[dev] > 0) {
        *out = g_cu_count[dev];
        return ANY4_OK;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return ANY4_E_HIP;
    if (dev >= 0 && dev < MAX_DEVICES)
        g_cu_count[dev] = cus;
    *out = cus;
    return ANY4_OK;
}

any4_status launched()
{
    return hipGetLastError() == hipSuccess ? ANY4_OK : ANY4_E_HIP;
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
    case ANY4_E_SHAPE: return "ANY4_E_SHAPE: unsupported sizes (negative size, odd K, g not a "
                              "positive multiple of 128, K % g != 0, or M > 16)";
    case ANY4_E_ALIGN: return "ANY4_E_ALIGN: a base pointer is not aligned as required";
    case ANY4_E_WORKSPACE: return "ANY4_E_WORKSPACE: workspace too small";
    case ANY4_E_HIP: return "ANY4_E_HIP: the HIP runtime reported an error";
    }
    return "any4: unknown status";
}

any4_status any4_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream)
{
    if (N < 0 || K < 0 || K % 2 != 0)
        return ANY4_E_SHAPE;
    if (N == 0 || K == 0)
        return ANY4_OK;
    if (!idx || !packed)
        return ANY4_E_NULL;
    if (!aligned(idx, 16) || !aligned(packed, 16))
        return ANY4_E_ALIGN;
    const size_t nout = static_cast<size_t>(N) * static_cast<size_t>(K / 2);
    const size_t threads = (nout + 15) / 16;
    const size_t blocks = (threads + PACK_THREADS - 1) / PACK_THREADS;
    if (blocks > 0x7FFFFFFFu)
        return ANY4_E_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_pack, dim3(static_cast<unsigned>(blocks)), dim3(PACK_THREADS), 0, stream,
                       idx, packed, nout);
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
    if (!packed || !lut || !alpha || !beta || !w)
        return ANY4_E_NULL;
    if (!aligned(packed, 16) || !aligned(lut, 16) || !aligned(w, 16) || !aligned(alpha, 2) ||
        !aligned(beta, 2))
        return ANY4_E_ALIGN;
    const size_t units = static_cast<size_t>(N) * static_cast<size_t>(K) / DQ_PER_THREAD;
    const size_t blocks = (units + DQ_THREADS - 1) / DQ_THREADS;
    if (blocks > 0x7FFFFFFFu)
        return ANY4_E_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_dequant, dim3(static_cast<unsigned>(blocks)), dim3(DQ_THREADS), 0, stream,
                       packed, lut, alpha, beta, w, K, g, units);
    return launched();
}

size_t any4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t g)
{
    (void)M;
    (void)N;
    (void)K;
    (void)g;
    return 0;
}

any4_status any4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    (void)workspace;
    if (M < 0 || M > 16 || N < 0 || !group_ok(K, g))
        return ANY4_E_SHAPE;
    if (N > 0x7FFFFFFF / 16 || K > 0x7FFFFFFF / 2 || N * (K / g) > 0x7FFFFFFF)
        return ANY4_E_SHAPE;
    if (M == 0 || N == 0)
        return ANY4_OK;
    if (!lut || !y || (K > 0 && (!x || !packed || !alpha || !beta)))
        return ANY4_E_NULL;
    if (!aligned(lut, 16) || !aligned(y, 2) ||
        (K > 0 && (!aligned(x, 16) || !aligned(packed, 16) || !aligned(alpha, 2) ||
                   !aligned(beta, 2))))
        return ANY4_E_ALIGN;
    if (workspace_bytes < any4_gemm_workspace_size(M, N, K, g))
        return ANY4_E_WORKSPACE;
    int cus = 0;
    if (cu_count(&cus) != ANY4_OK)
        return ANY4_E_HIP;
    const int ntiles = static_cast<int>((N + TILE_N - 1) / TILE_N);
    const int grid = ntiles < 2 * cus ? ntiles : 2 * cus;   // 64 KB of LDS: 2 per CU
    (void)hipGetLastError();
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K),
              gg = static_cast<int>(g);
#define ANY4_LAUNCH(MT)                                                                         \
    hipLaunchKernelGGL(k_gemm<MT>, dim3(grid), dim3(GEMM_THREADS), 0, stream, x, packed, lut,    \
                       alpha, beta, y, m, n, k, gg)
    if (M == 1)
        ANY4_LAUNCH(1);
    else if (M == 2)
        ANY4_LAUNCH(2);
    else if (M <= 4)
        ANY4_LAUNCH(4);
    else if (M <= 8)
        ANY4_LAUNCH(8);
    else
        ANY4_LAUNCH(16);
#undef ANY4_LAUNCH
    return launched();
}

}  // extern "C"
