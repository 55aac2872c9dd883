// libany4 -- any4 dequantize-GEMM for MI355X (gfx950, CDNA4).
//
// What is computed (the 10100.com any4 explainer): each weight is a 4-bit index
// into its row's 16-entry bf16 table (section 二), each contiguous group of g
// weights of a row has a scale alpha and an offset beta (step 1, "分组缩放"), so
// w = alpha * LUT_row[idx] + beta; the matmul y = x * W^T runs at decode batch
// sizes 1..16 (section 三).  Also here: the same product for plain int4 and for
// any2 and any3 (2- and 3-bit codes, the any4 paper's abstract), larger
// batches, and the quantiser that learns the tables (step 2, E-step /
// M-step).  The C ABI is declared in include/any4.h.
//
// Packed tile layout (written by k_pack, read by k_dequant and the GEMMs)
//   The weights are cut into tiles of 16 rows x 128 k.  A tile is 1 KB and is
//   one 16-byte load per lane of a wave64: lane l holds row (l % 16) of the
//   tile, k in [32*(l/16), 32*(l/16) + 32), two indices per byte, the even k
//   in the low nibble.  Tiles are stored row-block major: tile (b, c) of row
//   block b (rows 16b..16b+15) and k-chunk c (k 128c..128c+127) starts at byte
//   (b * K/128 + c) * 1024.  Rows past N are zero padding.  any2 tiles are the
//   same with four 2-bit codes per byte: 512 bytes, an 8-byte load per lane;
//   any3 tiles hold 16 six-bit pair indices per lane in 12 bytes: 768 bytes,
//   a 12-byte load per lane.
//
// Kernels
//   k_pack, k_pack2, k_pack3        idx[N][K] u8 -> tiles, one tile slot per thread.
//   k_dequant, k_dequant2, k_dequant3  w = bf16(fma(alpha, LUT[idx], beta)), one slot
//                          per thread, rows stored whole through LDS.
//   k_gemm_st              y = x * W^T for M <= 16 with one to four row blocks
//                          per CU: the weights stream once, decoded through
//                          table lookups in LDS into v_mfma_f32_16x16x32_bf16
//                          operands; K optionally split over workgroups.
//                          M = 17..48: two or three 16-row slices of x.
//   k_split_sum            y from the split partial sums, in split order.
//   k_gemm_km, k_gemm_kb   the same decode for more than four row blocks per CU.
//   k_gemm_big             M > 48 without a workspace: tiles dequantised into
//                          LDS, then MFMAs.  From M = 128 with a workspace the
//                          layer is dequantised into it (k_dequant*) and y is
//                          one hipBLASLt bf16 GEMM.
//   k_quantize_w           group scale + weighted k-means, one wave per row
//                          (k_quantize, one thread per row, for rows of more
//                          than 1024 groups).
//   k_read_probe           a streaming read (measurement only).
//   k_zero                 y = 0 when K = 0.
#include <hip/hip_runtime.h>

#include <hipblaslt/hipblaslt.h>
#include <cstdlib>
#include <mutex>
#include <deque>

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
// the 8 bytes of an any2 tile slot, non-temporal, in the low half of a u32x4
__device__ __forceinline__ u32x4_t load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
    return u32x4_t{v[0], v[1], 0u, 0u};
}
__device__ __forceinline__ u32x4_t load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
// the 12 bytes of an any3 tile slot, non-temporal, in the low three dwords
__device__ __forceinline__ u32x4_t load12_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 2);
    return u32x4_t{v[0], v[1], v[2], 0u};
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

// The decoded weights of a dequant workgroup (16 rows x DQ_WAVES chunks; the
// lane's 32 of row j, k-quarter kq of chunk wave wv, in out) go through LDS
// and are stored as whole rows: a wave's 16-byte stores then cover 1 KB of
// one row instead of 16 rows' 16-byte pieces.  Called by every thread (it
// holds a barrier); `live`: the lane decoded something.
constexpr int DQ_RP = DQ_WAVES * 16 + 1;   // 16-byte pieces per staged row (+1: banks)
__device__ __forceinline__ void dq_store_rows(u32x4_t* so, const u32x4_t (&out)[4], bool live,
                                              int wv, int j, int kq, int b, int cg0, int Kc,
                                              int N, int K, uint16_t* __restrict__ w)
{
    if (live) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            so[j * DQ_RP + wv * 16 + kq * 4 + q] = out[q];
    }
    __syncthreads();
    // piece pc of row r: k = (cg0 + pc/16) * 128 + (pc%16) * 8
    const int nch = min(DQ_WAVES, Kc - cg0);
#pragma unroll
    for (int i = 0; i < TILE_ROWS * 16 / 64; ++i) {
        const int pi = threadIdx.x + i * 64 * DQ_WAVES;
        const int r = pi / (DQ_WAVES * 16);
        const int pc = pi - r * (DQ_WAVES * 16);
        const int nr = b * TILE_ROWS + r;
        if (nr < N && pc < nch * 16)
            *reinterpret_cast<u32x4_t*>(w + static_cast<size_t>(nr) * K + cg0 * TILE_K + pc * 8) =
                so[r * DQ_RP + pc];
    }
}

// w[n][k] = bf16(fma(alpha, LUT[idx], beta)).  The workgroup's 16 table rows
// are widened to fp32 in LDS; each lane decodes the 32 weights of its tile
// slot (a row's quarter of the wave's 128 k).  The decoded rows go through
// LDS so that the stores are whole rows: a wave's 16-byte stores cover 1 KB
// of one row (the workgroup's 4 chunks), not 16 rows' 16-byte pieces.
// i4: plain int4, the code itself is the value (the table 0..15; lut unread).
__global__ __launch_bounds__(64 * DQ_WAVES) void k_dequant(const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ lut,
                                                          const uint16_t* __restrict__ alpha,
                                                          const uint16_t* __restrict__ beta,
                                                          uint16_t* __restrict__ w, int N, int K,
                                                          int g, int i4)
{
    __shared__ float sl[TILE_ROWS * 16];
    __shared__ u32x4_t so[TILE_ROWS * DQ_RP];
    const int Kc = K / TILE_K;
    const int cgroups = (Kc + DQ_WAVES - 1) / DQ_WAVES;
    const int b = blockIdx.x / cgroups;
    const int cg0 = (blockIdx.x % cgroups) * DQ_WAVES;   // the workgroup's first chunk
    const int wv = threadIdx.x >> 6;
    const int c = cg0 + wv;
    {
        const int t = threadIdx.x;   // 256 threads: row t/16, entry t%16
        const int n = b * TILE_ROWS + (t >> 4);
        sl[t] = i4 ? static_cast<float>(t & 15)
                   : n < N ? bf16_to_f32(lut[static_cast<size_t>(n) * 16 + (t & 15)]) : 0.f;
    }
    __syncthreads();
    const int l = threadIdx.x & 63;
    const int j = l & 15;
    const int kq = l >> 4;
    const int n = b * TILE_ROWS + j;
    const bool live = c < Kc && n < N;
    u32x4_t out[4];
    if (live) {
        const int k0 = c * TILE_K + kq * 32;
        const int G = K / g;
        const float a = bf16_to_f32(alpha[static_cast<size_t>(n) * G + k0 / g]);
        const float bt = bf16_to_f32(beta[static_cast<size_t>(n) * G + k0 / g]);
        const u32x4_t p = *reinterpret_cast<const u32x4_t*>(
            packed + (static_cast<size_t>(b) * Kc + c) * TILE_BYTES + l * 16);
        const float* L = sl + j * 16;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint32_t byte = (p[q >> 2] >> (8 * (q & 3))) & 0xFFu;
            const float lo = fmaf(a, L[byte & 15u], bt);
            const float hi = fmaf(a, L[byte >> 4], bt);
            out[q >> 2][q & 3] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
        }
    }
    dq_store_rows(so, out, live, wv, j, kq, b, cg0, Kc, N, K, w);
}

// ---- any2 (2-bit codes) -----------------------------------------------------
// Tiles of 16 rows x 128 k, 512 bytes: byte 8l + i of tile (b, c) holds row
// 16b + l%16, codes k = 128c + 32(l/16) + 4i .. +3 in bits 0-1, 2-3, 4-5, 6-7.
// One 8-byte slot per lane of a wave64; each slot is exactly the 32 k of the
// lane's four MFMA B operands.
__global__ __launch_bounds__(PACK_THREADS) void k_pack2(const uint8_t* __restrict__ idx,
                                                        uint8_t* __restrict__ packed, int N,
                                                        int K, uint32_t slots)
{
    const uint32_t sidx = blockIdx.x * PACK_THREADS + threadIdx.x;   // 8-byte slot
    if (sidx >= slots)
        return;
    const int Kc = K / TILE_K;
    const uint32_t tile = sidx / 64;
    const int l = static_cast<int>(sidx % 64);
    const int b = static_cast<int>(tile / Kc);
    const int c = static_cast<int>(tile % Kc);
    const int n = b * TILE_ROWS + (l & 15);
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    u32x2_t out = {0u, 0u};
    if (n < N) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
            idx + static_cast<size_t>(n) * K + c * TILE_K + (l >> 4) * 32);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t v = src[h];   // 16 codes, one per byte
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = v[q] & 0x03030303u;   // codes 4q' .. 4q'+3 of this dword
                const uint32_t byte = (w & 3u) | ((w >> 6) & 0xCu) | ((w >> 12) & 0x30u) |
                                      ((w >> 18) & 0xC0u);
                out[h] |= byte << (8 * q);
            }
        }
    }
    *reinterpret_cast<u32x2_t*>(packed + static_cast<size_t>(sidx) * 8) = out;
}

__global__ __launch_bounds__(64 * DQ_WAVES) void k_dequant2(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ lut,
                                                           const uint16_t* __restrict__ alpha,
                                                           const uint16_t* __restrict__ beta,
                                                           uint16_t* __restrict__ w, int N, int K,
                                                           int g)
{
    __shared__ float sl[TILE_ROWS * 4];
    __shared__ u32x4_t so[TILE_ROWS * DQ_RP];
    const int Kc = K / TILE_K;
    const int cgroups = (Kc + DQ_WAVES - 1) / DQ_WAVES;
    const int b = blockIdx.x / cgroups;
    const int cg0 = (blockIdx.x % cgroups) * DQ_WAVES;
    const int wv = threadIdx.x >> 6;
    const int c = cg0 + wv;
    if (threadIdx.x < TILE_ROWS * 4) {   // row t/4, entry t%4
        const int t = threadIdx.x;
        const int n = b * TILE_ROWS + (t >> 2);
        sl[t] = n < N ? bf16_to_f32(lut[static_cast<size_t>(n) * 16 + (t & 3)]) : 0.f;
    }
    __syncthreads();
    const int l = threadIdx.x & 63;
    const int j = l & 15;
    const int n = b * TILE_ROWS + j;
    const bool live = c < Kc && n < N;
    u32x4_t out[4];
    if (live) {
        const int k0 = c * TILE_K + (l >> 4) * 32;
        const int G = K / g;
        const float a = bf16_to_f32(alpha[static_cast<size_t>(n) * G + k0 / g]);
        const float bt = bf16_to_f32(beta[static_cast<size_t>(n) * G + k0 / g]);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t p = *reinterpret_cast<const u32x2_t*>(
            packed + (static_cast<size_t>(b) * Kc + c) * (TILE_BYTES / 2) + l * 8);
        const float* L = sl + j * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {   // byte i: codes 4i .. 4i+3
            const uint32_t byte = (p[i >> 2] >> (8 * (i & 3))) & 0xFFu;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float lo = fmaf(a, L[(byte >> (4 * t)) & 3u], bt);
                const float hi = fmaf(a, L[(byte >> (4 * t + 2)) & 3u], bt);
                const int d = 2 * i + t;
                out[d >> 2][d & 3] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
            }
        }
    }
    dq_store_rows(so, out, live, wv, j, l >> 4, b, cg0, Kc, N, K, w);
}

// ---- any3 (3-bit codes) -----------------------------------------------------
// Tiles of 16 rows x 128 k, 768 bytes: the 12-byte slot of lane l (bytes
// 12l .. 12l+11 of tile (b, c)) holds row 16b + l%16, codes
// k = 128c + 32(l/16) + 0..31 as 16 pair indices P_i = code[2i] | code[2i+1] << 3.
// Byte j < 12 holds P_j in bits 0-5 and, in bits 6-7, bits 2(j/4)..2(j/4)+1
// of P_{12 + j%4}.  Dword s < 3 of a slot is thus the pair bytes of the
// lane's MFMA B operand s, and the fourth operand's pair bytes are gathered
// from the top bits.

// any3: the pair indices 12..15 of a 12-byte slot, one per byte, gathered
// from bits 6-7 of the slot's bytes (pair 12 + t: bits 0-1 from byte t, 2-3
// from byte 4 + t, 4-5 from byte 8 + t).  Bits 6-7 of each result byte are
// left undefined (every reader masks them or ignores them): two bit-field
// inserts place the three parts at bits 2-7, one shift moves them down.
// (a & mask) | (b & ~mask) as one v_bfi_b32: written out in C, the compiler
// folds the two inserts below into three masks and an or3 (two more VALU)
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t any3_top_pairs(const u32x4_t& p)
{
    return bfi(0xC0C0C0C0u, p[2], bfi(0x30303030u, p[1] >> 2, p[0] >> 4)) >> 2;
}

__device__ __forceinline__ uint32_t pack3_pair(uint32_t codes2)   // two code bytes -> P
{
    return (codes2 & 7u) | ((codes2 >> 5) & 0x38u);
}

__global__ __launch_bounds__(PACK_THREADS) void k_pack3(const uint8_t* __restrict__ idx,
                                                        uint8_t* __restrict__ packed, int N,
                                                        int K, uint32_t slots)
{
    const uint32_t sidx = blockIdx.x * PACK_THREADS + threadIdx.x;   // 12-byte slot
    if (sidx >= slots)
        return;
    const int Kc = K / TILE_K;
    const uint32_t tile = sidx / 64;
    const int l = static_cast<int>(sidx % 64);
    const int b = static_cast<int>(tile / Kc);
    const int c = static_cast<int>(tile % Kc);
    const int n = b * TILE_ROWS + (l & 15);
    uint32_t out[3] = {0u, 0u, 0u};
    if (n < N) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
            idx + static_cast<size_t>(n) * K + c * TILE_K + (l >> 4) * 32);
        const u32x4_t v0 = src[0], v1 = src[1];
        const uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t P[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)   // codes 2i, 2i+1: bytes 2(i%2), +1 of dword i/2
            P[i] = pack3_pair(w[i >> 1] >> (16 * (i & 1)));
#pragma unroll
        for (int jb = 0; jb < 12; ++jb) {
            const uint32_t byte = P[jb] | (((P[12 + (jb & 3)] >> (2 * (jb >> 2))) & 3u) << 6);
            out[jb >> 2] |= byte << (8 * (jb & 3));
        }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(packed + static_cast<size_t>(sidx) * 12);
    dst[0] = out[0];
    dst[1] = out[1];
    dst[2] = out[2];
}

__global__ __launch_bounds__(64 * DQ_WAVES) void k_dequant3(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ lut,
                                                           const uint16_t* __restrict__ alpha,
                                                           const uint16_t* __restrict__ beta,
                                                           uint16_t* __restrict__ w, int N, int K,
                                                           int g)
{
    __shared__ float sl[TILE_ROWS * 8];
    __shared__ u32x4_t so[TILE_ROWS * DQ_RP];
    const int Kc = K / TILE_K;
    const int cgroups = (Kc + DQ_WAVES - 1) / DQ_WAVES;
    const int b = blockIdx.x / cgroups;
    const int cg0 = (blockIdx.x % cgroups) * DQ_WAVES;
    const int wv = threadIdx.x >> 6;
    const int c = cg0 + wv;
    if (threadIdx.x < TILE_ROWS * 8) {   // row t/8, entry t%8
        const int t = threadIdx.x;
        const int n = b * TILE_ROWS + (t >> 3);
        sl[t] = n < N ? bf16_to_f32(lut[static_cast<size_t>(n) * 16 + (t & 7)]) : 0.f;
    }
    __syncthreads();
    const int l = threadIdx.x & 63;
    const int j = l & 15;
    const int n = b * TILE_ROWS + j;
    const bool live = c < Kc && n < N;
    u32x4_t out[4];
    if (live) {
        const int k0 = c * TILE_K + (l >> 4) * 32;
        const int G = K / g;
        const float a = bf16_to_f32(alpha[static_cast<size_t>(n) * G + k0 / g]);
        const float bt = bf16_to_f32(beta[static_cast<size_t>(n) * G + k0 / g]);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            packed + (static_cast<size_t>(b) * Kc + c) * (TILE_BYTES * 3 / 4) + l * 12);
        const u32x4_t p = {src[0], src[1], src[2], 0u};
        const uint32_t top = any3_top_pairs(p);
        const float* L = sl + j * 8;
#pragma unroll
        for (int i = 0; i < 16; ++i) {   // pair i: codes 2i, 2i+1
            const uint32_t d = i < 12 ? p[i >> 2] : top;
            const uint32_t P = (d >> (8 * (i & 3))) & 0x3Fu;
            const float lo = fmaf(a, L[P & 7u], bt);
            const float hi = fmaf(a, L[P >> 3], bt);
            out[i >> 2][i & 3] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
        }
    }
    dq_store_rows(so, out, live, wv, j, l >> 4, b, cg0, Kc, N, K, w);
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

// Two kernels compute y = x * W^T, both persistent and k-major: about one
// workgroup per CU owns 16-row blocks r, r+G, r+2G, ... of W and decodes up
// to four of them together, chunk (128 k) by chunk, against the same x
// operands; the 8 waves split K and meet in LDS at the end.
//
//   k_gemm_km   K <= 4096: a wave's 4 chunks, fully unrolled.
//   k_gemm_kb   any K: a wave's K/1024 chunks in steps of the ring depth.
//
// Decode.  A packed byte (two indices) selects one dword of a pair table in
// LDS: entry (hi << 4 | lo) holds the table values (L[lo], L[hi]) as two
// 16-bit halves, in the order of an MFMA B operand dword.  The table of a row
// block has 32 slots per entry (slot = lane % 32, row = slot % 16); a wave64
// LDS read is served as two halves of 32 lanes, so every lane reads its own
// bank: no conflicts.  Entry e of a table sits at byte e*256 (+128 for the
// second table of a 64 KB region), so the read address is one v_perm of the
// packed dword.
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
// loop bodies are straight-line apart from uniform branches, so the ring
// survives the loop.
constexpr int GW = 8;                   // waves per workgroup

// Weight formats of the GEMM kernels: the any4 table path, plain int4 (the
// code is the value), any2 (2-bit codes, four per byte, 512-byte tiles; a
// byte looks up four table values at once) and any3 (3-bit codes, a 6-bit
// pair index per byte plus four pairs spread over the bytes' top bits,
// 768-byte tiles; looked up like any4 pairs).
constexpr int FMT_ANY4 = 0;
constexpr int FMT_INT4 = 1;
constexpr int FMT_ANY2 = 2;
constexpr int FMT_ANY3 = 3;
constexpr int tile_bytes(int fmt)
{
    return fmt == FMT_ANY2 ? TILE_BYTES / 2 : fmt == FMT_ANY3 ? TILE_BYTES * 3 / 4 : TILE_BYTES;
}
constexpr int GT = 64 * GW;
constexpr int TAB_BYTES = 256 * 256;    // 256 entries x 2 tables x 32 slots x 4 B
constexpr int MAX_G = 512;              // K/g: the alpha/beta staging of k_gemm_kb

struct GemmArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* lut;
    const uint16_t* alpha;
    const uint16_t* beta;
    uint16_t* y;
    int M, N, K, g;
    float* ws;          // split-K partial sums (k_gemm_st), or null: no split
    size_t ws_bytes;
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

// Build the pair table of one row block, whose entry 0 starts at dword
// `tab_dw` of LDS (entries 64 dwords apart), from its 16 table rows, staged
// in LDS at `lut_off` as [16 rows][16] 16-bit values.  Thread t of the W*64
// writes slot t % 32 (row (t % 32) % 16) of the entries lo + 16*hi,
// lo = (t / 32) % 16, for its share of the 16 hi.
//
// any3 (A3): entry e holds (L[e & 7], L[(e >> 3) & 7]): the low 6 bits of the
// byte are the pair of 3-bit codes and bits 6-7 select one of four identical
// copies, so a byte whose top bits carry other data needs no masking.
template <int W, bool A3 = false>
__device__ __forceinline__ void build_table(uint8_t* smem, uint32_t lut_off, uint32_t tab_dw,
                                            int tid)
{
    constexpr int HPT = 128 / W;   // hi values per thread
    const int st = tid & 31;
    const int lo = (tid >> 5) & 15;
    const int h0 = (tid >> 9) * HPT;
    const uint32_t row = lut_off + (st & 15) * 32;
    const u32x4_t q0 = lds_at<u32x4_t>(smem, row);
    const u32x4_t q1 = lds_at<u32x4_t>(smem, row + 16);
    const uint32_t ll = lds_at<uint16_t>(smem, row + 2 * (A3 ? lo & 7 : lo));
    const uint32_t Lw[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
    uint32_t* tw = reinterpret_cast<uint32_t*>(smem) + tab_dw + lo * 64 + st;
    if constexpr (A3) {
        static_assert(HPT == 16, "one thread per (slot, lo) pair");
        // entry hi << 4 | lo: the second code is (2*hi + lo/8) & 7, the
        // half (lo/8) of dword hi & 3 of the row
        const uint32_t sel = (lo >> 3) ? 0x07060100u : 0x05040100u;
#pragma unroll
        for (int hi = 0; hi < 16; ++hi)
            tw[hi * 16 * 64] = __builtin_amdgcn_perm(Lw[hi & 3], ll, sel);
    } else if constexpr (HPT == 16) {
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

// any2: the quad table of one row block.  Entry e (a byte of four 2-bit codes
// c_s = (e >> 2s) & 3) holds (L[c0] | L[c1] << 16, L[c2] | L[c3] << 16): the
// two B-operand dwords of those four weights.  16 slots per entry (slot =
// row), 8 bytes each: entry e at byte e*256 (+128 for the second table of a
// 64 KB region) + slot*8, so one 64-bit read decodes four weights.  Thread t
// of the W*64 writes slot t % 16 of entries t / 16 + (64*W/16)*i.
template <int W>
__device__ __forceinline__ void build_table2(uint8_t* smem, uint32_t lut_off, uint32_t tab_off,
                                             int tid)
{
    constexpr int EPT = 256 * 16 / (64 * W);   // entries per thread
    const int st = tid & 15;
    const uint32_t row = lut_off + st * 32;
    const uint32_t A = lds_at<uint32_t>(smem, row);       // L0 | L1 << 16
    const uint32_t B = lds_at<uint32_t>(smem, row + 4);   // L2 | L3 << 16
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const uint32_t e = static_cast<uint32_t>(tid >> 4) + i * (64 * W / 16);
        // byte selector of v_perm(B, A): bytes 0-3 are A's, 4-7 are B's
        auto sel = [](uint32_t qa, uint32_t qb) {
            return (2 * qa) | ((2 * qa + 1) << 8) | ((2 * qb) << 16) | ((2 * qb + 1) << 24);
        };
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = {__builtin_amdgcn_perm(B, A, sel(e & 3, (e >> 2) & 3)),
                           __builtin_amdgcn_perm(B, A, sel((e >> 4) & 3, e >> 6))};
        lds_at<u32x2_t>(smem, tab_off + e * 256 + st * 8) = v;
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

// floor(a / d) for 0 <= a < 2^22 from inv = 1/d rounded to fp32: (a + 1/2)/d
// lies at least 1/(2d) from an integer and the product's error is below
// (a + 1/2)/d * 2^-23, so the truncation is exact.
__device__ __forceinline__ int small_div(int a, float inv)
{
    return static_cast<int>((static_cast<float>(a) + 0.5f) * inv);
}

// store_pairs for a staged range of groups: of the 8 values of piece q
// (elements 8q..8q+7 of the block's [16][G] arrays), those of groups
// gbase..gbase+GS-1, stored as [group - gbase][row].  inv_G = 1/G in fp32
// (8q < 2^22).
__device__ __forceinline__ void store_pairs_range(uint8_t* smem, uint32_t base, int q, int G,
                                                  float inv_G, int gbase, int GS,
                                                  const u32x4_t& qa, const u32x4_t& qb)
{
    int row = small_div(8 * q, inv_G);
    int grp = 8 * q - row * G;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const int gi = grp - gbase;
        if (gi >= 0 && gi < GS && row < 16)
            lds_at<uint32_t>(smem, base + (gi * 16 + row) * 4) =
                __builtin_amdgcn_perm(qb[i >> 1], qa[i >> 1], sel);
        if (++grp == G) {
            grp = 0;
            ++row;
        }
    }
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

// ---- k_gemm_km: k-major, every row block of a workgroup decoded together --
//
// A workgroup owns the row blocks r, r+Gs, r+2Gs, ... (at most KM_MAX_BLK)
// and takes them NBG at a time (a group): the pair tables of all NBG blocks
// of a group are built once, then each wave walks its KM_C chunks of 128 k
// and, for each chunk, decodes that chunk's tile of every block of the group
// with the same x operands.  The loop has no barrier: the tables stay put
// for the whole group, and the waves meet only at the group's end, where
// their partial sums are added in LDS.
//
// Dequantisation.  Every weight is formed as w = bf16(fp32(alpha*L + beta))
// before it enters the MFMA, the same value any4_dequant writes, so y is the
// product over the dequantised matrix up to fp32 summation order.  The
// tables hold L as f16, scaled per row by 2^-s so that the row's largest
// finite magnitude lies in [2^14, 2^15): every value within 2^31 of it is
// exact in f16, and alpha*2^s * (L*2^-s) = alpha*L exactly.  v_fma_mix_f32
// takes an f16 half of the looked-up dword directly, so a dword of two
// weights costs two fma_mix and one v_cvt_pk_bf16_f32.
//
// x: for M <= 2 the whole of x (<= 16 KB) is copied to LDS in the prologue
// and each pair's operands are read from there (lanes of rows m >= M read
// row M-1: those MFMA rows are never stored).  For larger M they travel in
// the ring with the tiles: a chunk's 4 operand loads are issued right after the chunk's last
// tile (its slot is free by then: the chunk DS chunks earlier, which used it,
// has just been decoded), so waiting for them never waits for a later chunk.
//
// Decode: two tiles at a time (two blocks of one chunk, or two chunks): the
// 32 table lookups, the dequantisation, then the two MFMA chains
// interleaved, so the chains' latencies overlap; the next pair's lookups are
// issued before the current pair is dequantised.
//
// Prologue: the first ring loads go out with the staging loads; the rest are
// spread over the table builds, so the builds overlap the first tiles'
// latency instead of waiting behind a full ring.
//
// LDS:
//   [0, TABS)  pair tables: table b sits in 64 KB region b/2, half b%2, entry
//              e at byte e*256 + (b%2)*128 + slot*4 (the x staging of the
//              prologue and the partial sums of a group's end reuse it)
//   ZERO       256 zero bytes at the start of the next 64 KB region: a dead
//              tile (a chunk past K) reads its "table entries" here, so that
//              an inf or NaN in a table entry no weight uses cannot reach y
//   AB         [NBG][G <= 32][16 rows] (alpha | beta << 16) dwords
//   LUTS       [NBG][16 rows][16] f16, each row scaled by 2^-s
//   SCL        [NBG][16 rows] int: the row scale exponents s
//   XS         (M <= 2) x as [M][K] bf16
constexpr int KM_C = 4;                              // chunks per wave
constexpr int KM_MAX_K = GW * KM_C * TILE_K;         // 4096
constexpr int KM_MAX_G = KM_MAX_K / TILE_K;          // g >= 128
constexpr int KM_MAX_BLK = 8;                        // row blocks per workgroup

template <int NBG>
struct KmCfg {
    static constexpr int TABS = ((NBG + 1) / 2) * 65536;
    static constexpr int ZERO = TABS;   // 256 zero bytes: the table reads of dead tiles
    static constexpr int AB_BLK = KM_MAX_G * 16 * 4;
    static constexpr int AB = ZERO + 256;
    static constexpr int LUTS = AB + NBG * AB_BLK;
    static constexpr int SCL = LUTS + NBG * 512;     // [NBG][16 rows] int: row scale exponents
    static constexpr int XS = SCL + NBG * 64;        // x as [M <= 2][K <= 4096] bf16
    static constexpr int LDS = XS + 2 * KM_MAX_K * 2;
    static constexpr int GS = KM_C * NBG;                                  // tiles per wave per group
    static constexpr int D = GS > 8 ? (GS % 8 == 0 ? 8 : GS / 2) : GS;   // ring depth in tiles
    static constexpr int DS = D / NBG;                                     // ... in chunks
    static_assert(GS % D == 0 && D % NBG == 0, "the ring holds whole chunks of a group");
};

// (lane part | uniform part): either part may be OOR; valid parts are < 2^31.
__device__ __forceinline__ uint32_t off2(uint32_t lane_part, uint32_t uni)
{
    return (lane_part | (uni & OOR)) + (uni & ~OOR);
}

// Largest biased exponent over the finite bf16 values of a row, whose 16
// values are split over lanes l and l^1 (8 each in the 4 dwords of q).
__device__ __forceinline__ int row_emax(const u32x4_t& q)
{
    int e = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e0 = (q[i] >> 7) & 0xFF;
        const int e1 = (q[i] >> 23) & 0xFF;
        e = max(e, e0 == 0xFF ? 0 : e0);
        e = max(e, e1 == 0xFF ? 0 : e1);
    }
    return max(e, __shfl_xor(e, 1));
}

// Row scale exponent s: the largest finite magnitude times 2^-s lies in
// [2^14, 2^15); at least -60 (rows of values below 2^-74).
__device__ __forceinline__ int lut_scale(const u32x4_t& q)
{
    return max(row_emax(q) - 141, -60);
}

// 8 bf16 table values -> 8 f16 values times 2^-s
__device__ __forceinline__ u32x4_t lut_to_f16(const u32x4_t& q, int s)
{
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_ldexpf(bf16_to_f32(q[i] & 0xFFFFu), -s);
        const float hi = __builtin_ldexpf(bf16_to_f32(q[i] >> 16), -s);
        const h2_t h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
        r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

// bf16(a*L + b) for the two f16 table values of a pair dword, packed
__device__ __forceinline__ uint32_t deq_pair(uint32_t d, float a, float b)
{
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    const h2_t l = __builtin_bit_cast(h2_t, d);
    const f2_t w = {fmaf(a, static_cast<float>(l.x), b), fmaf(a, static_cast<float>(l.y), b)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf2_t));
}

// int4 (no table): the four bytes of a packed dword give the B-operand
// dwords bf16(a*lo + b) | bf16(a*hi + b) << 16, lo/hi the byte's nibbles
__device__ __forceinline__ u32x4_t deq_int4(uint32_t d, float a, float b)
{
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    // The masks go through asm so that the byte conversions below stay single
    // v_cvt_f32_ubyte<jb> instructions: with the mask visible, the compiler
    // folds each into a bit-field extract plus a conversion.
    uint32_t lo, hi;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(d));
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(d >> 4));
    u32x4_t r;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const f2_t w = {fmaf(a, static_cast<float>((lo >> (8 * jb)) & 0xFFu), b),
                        fmaf(a, static_cast<float>((hi >> (8 * jb)) & 0xFFu), b)};
        r[jb] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf2_t));
    }
    return r;
}

__device__ __forceinline__ u32x4_t deq_quad(const u32x4_t& q, float a, float b)
{
    return u32x4_t{deq_pair(q[0], a, b), deq_pair(q[1], a, b), deq_pair(q[2], a, b),
                   deq_pair(q[3], a, b)};
}

template <int MT, int NBG, int FMT>
__global__ __launch_bounds__(GT) void k_gemm_km(const GemmArgs args)
{
    constexpr bool I4 = FMT == FMT_INT4;
    constexpr bool A2 = FMT == FMT_ANY2;
    constexpr bool A3 = FMT == FMT_ANY3;
    constexpr uint32_t TB = tile_bytes(FMT);
    using Cfg = KmCfg<NBG>;
    constexpr int C = KM_C;
    constexpr int GS = Cfg::GS;
    constexpr int D = Cfg::D;
    constexpr int DS = Cfg::DS;
    constexpr int VC = MT < 4 ? MT : 4;
    constexpr bool XSTREAM = MT > 2;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int kq = lane >> 4;
    const int Kc = K / TILE_K;
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = K / g;
    const int Gs = gridDim.x;
    const int r = blockIdx.x;
    const int nblk = r < NB ? (NB - 1 - r) / Gs + 1 : 0;
    const int ngroups = (nblk + NBG - 1) / NBG;
    const int cbase = wave * C;

    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TB);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, static_cast<uint32_t>(N) * 32);
    // alpha/beta are read with 16-byte loads: the range is rounded up to 16 B
    // (the 16-byte granule holding a valid byte never leaves that byte's page
    // when the base is 16-byte aligned); the extra values only reach rows >= N.
    const uint32_t ab_range = (static_cast<uint32_t>(N) * G * 2 + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, ab_range);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, ab_range);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // ---- staging of a group: wave b < NBG fetches block b's 16 table rows
    // (lanes < 32) and its alpha and beta (lanes < 2G, 16 B each)
    const uint32_t lut_lane = lane < 32 ? static_cast<uint32_t>(lane) * 16 : OOR;
    const uint32_t ab_lane = lane < 2 * G ? static_cast<uint32_t>(lane) * 16 : OOR;
    auto stage_load = [&](int gi, u32x4_t& lq, u32x4_t& aq, u32x4_t& bq) {
        const int blk = gi * NBG + wave;
        const bool live = wave < NBG && blk < nblk;
        const uint32_t b = static_cast<uint32_t>(r + blk * Gs);
        if constexpr (!I4)
            lq = load16(rl, off2(lut_lane, live ? b * 512 : OOR));
        else
            lq = u32x4_t{0u, 0u, 0u, 0u};
        const uint32_t ao = off2(ab_lane, live ? b * (G * 32) : OOR);
        aq = load16(ra, ao);
        bq = load16(rb, ao);
    };
    auto stage_store = [&](const u32x4_t& lq, const u32x4_t& aq, const u32x4_t& bq) {
        // table rows as f16, scaled by 2^-s (s per row: the largest finite
        // magnitude lands in [2^14, 2^15)), so every value within 2^31 of the
        // row's largest is exact; the decode multiplies alpha by 2^s
        int sc = 0;
        u32x4_t lh = lq;
        if constexpr (!I4) {
            sc = lut_scale(lq);   // all lanes: pairs of lanes share a row
            lh = lut_to_f16(lq, sc);
        }
        if (wave < NBG) {
            if (!I4 && lane < 32) {
                lds_at<u32x4_t>(smem, Cfg::LUTS + wave * 512 + lane * 16) = lh;
                if ((lane & 1) == 0)
                    lds_at<int>(smem, Cfg::SCL + (wave * 16 + (lane >> 1)) * 4) = sc;
            }
            if (lane < 2 * G)
                store_pairs(smem, Cfg::AB + wave * Cfg::AB_BLK, lane, G, aq, bq);
        }
    };
    auto build = [&](int bb) {
        if constexpr (A2)
            build_table2<GW>(smem, Cfg::LUTS + bb * 512, (bb >> 1) * 65536 + (bb & 1) * 128, tid);
        else if constexpr (!I4)
            build_table<GW, A3>(smem, Cfg::LUTS + bb * 512, (bb >> 1) * 16384 + (bb & 1) * 32,
                                tid);
    };

    // ---- ring: tile v of group gi is chunk cbase + v / NBG of block
    // gi*NBG + v % NBG (weights are streamed once: non-temporal loads); with
    // XSTREAM, the x operands of chunk s of a group follow its first tile
    u32x4_t pb[D];
    u32x4_t xq[XSTREAM ? DS : 1][4];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * (TB / 64);
    const uint32_t x_lane = j < M ? static_cast<uint32_t>(j * K + kq * 32) * 2 : OOR;
    auto issue = [&](int gi, int uu) {
        const int gg = gi + uu / GS;
        const int v = uu % GS;
        const int blk = gg * NBG + v % NBG;
        const int c = cbase + v / NBG;
        const bool live = blk < nblk && c < Kc;
        // computed unconditionally and pushed out of range with one OR: a
        // select here would become a branch around the load
        const uint32_t uo =
            (static_cast<uint32_t>(r + blk * Gs) * static_cast<uint32_t>(Kc) + c) * TB |
            (static_cast<uint32_t>(!live) << 31);
        pb[uu % D] = A2   ? load8_nt(rp, off2(tile_lane, uo))
                     : A3 ? load12_nt(rp, off2(tile_lane, uo))
                          : load16_nt(rp, off2(tile_lane, uo));
        if constexpr (XSTREAM) {
            if (v % NBG == NBG - 1) {
                const bool xl = gg < ngroups && c < Kc;
                const uint32_t xc =
                    static_cast<uint32_t>(c) * TILE_K * 2 | (static_cast<uint32_t>(!xl) << 31);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    xq[(uu / NBG) % DS][s4] = load16(rx, off2(x_lane, xc) + s4 * 16);
            }
        }
    };

    // ---- prologue
    u32x4_t lq, aq, bq;
    stage_load(0, lq, aq, bq);
    // x (M <= 2): the whole of x to LDS, two 16-byte pieces per thread
    u32x4_t xc16[2];
    const uint32_t xbytes = static_cast<uint32_t>(M) * K * 2;
    if constexpr (!XSTREAM) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * GT) * 16;
            xc16[i] = load16(rx, o < xbytes ? o : OOR);
        }
    }
    constexpr int R0 = D < 2 ? D : 2;   // ring loads issued with the staging loads
#pragma unroll
    for (int u = 0; u < R0; ++u)
        issue(0, u);
    if (tid < 16)
        lds_at<u32x4_t>(smem, Cfg::ZERO + tid * 16) = u32x4_t{0u, 0u, 0u, 0u};
    stage_store(lq, aq, bq);
    if constexpr (!XSTREAM) {
        // past x the region is zeroed: chunks past K read it (their weights
        // are zero, and 0 * NaN left over in LDS would not be)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * GT) * 16;
            lds_at<u32x4_t>(smem, Cfg::XS + o) = o < xbytes ? xc16[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();
    {
        constexpr int PER = (D - R0 + NBG - 1) / NBG;   // ring loads per table build
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb) {
            build(bb);
#pragma unroll
            for (int u = R0 + bb * PER; u < R0 + (bb + 1) * PER && u < D; ++u)
                issue(0, u);
        }
    }
    __syncthreads();

    // the lane's slot in a table entry (any2: 16 slots of 8 bytes)
    const uint32_t slot4 = A2 ? static_cast<uint32_t>(lane & 15) * 8 : static_cast<uint32_t>(lane & 31) * 4;
    const uint32_t s1[2] = {slot4, slot4 | 0x10000u};   // region 0 / region 1
    uint32_t ab_c[C];   // LDS offset of this lane's (alpha, beta) pair, block 0
#pragma unroll
    for (int ci = 0; ci < C; ++ci)
        ab_c[ci] = Cfg::AB + ((((cbase + ci) * TILE_K) / g) * 16 + j) * 4;

    constexpr int NA = NBG == 1 ? 2 : 1;   // one block: two chains, added at the end
    f32x4_t acc[NBG][NA];
#pragma unroll
    for (int bb = 0; bb < NBG; ++bb)
#pragma unroll
        for (int h = 0; h < NA; ++h)
            acc[bb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int rsc[NBG];   // scale exponent of this lane's row in each block's table
    auto load_scales = [&]() {
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb)
            rsc[bb] = I4 ? 0 : lds_at<int>(smem, Cfg::SCL + (bb * 16 + j) * 4);
    };
    load_scales();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);
    auto reduce_store = [&](int gi) {   // after a barrier: tables are free
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb) {
            f32x4_t t = acc[bb][0];
            if constexpr (NA > 1)
                t += acc[bb][NA - 1];
            red[(bb * GW + wave) * 64 + lane] = t;
        }
        __syncthreads();
        const int blk = gi * NBG + wave;
        if (wave < NBG && blk < nblk)
            store_block<MT, GW>(red + wave * GW * 64, args.y, lane, M, N,
                                (r + blk * Gs) * TILE_ROWS);
    };

    u32x4_t lqn, aqn, bqn;
    for (int gi = 0; gi < ngroups; ++gi) {
        if (gi > 0) {
            __syncthreads();
            reduce_store(gi - 1);
            stage_store(lqn, aqn, bqn);
            __syncthreads();
#pragma unroll
            for (int bb = 0; bb < NBG; ++bb)
                build(bb);
            __syncthreads();
            load_scales();
#pragma unroll
            for (int bb = 0; bb < NBG; ++bb)
#pragma unroll
                for (int h = 0; h < NA; ++h)
                    acc[bb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        stage_load(gi + 1, lqn, aqn, bqn);
        // Decode, software-pipelined over pairs of tiles: the 32 table lookups
        // (and two alpha/beta reads) of the next pair are issued before the
        // current pair is dequantised, so their LDS latency is covered by the
        // current pair's VALU work.
        u32x4_t bwp[2][2][4];
        uint32_t prp[2][2];
        auto fetch = [&](int u0, u32x4_t (&bw)[2][4], uint32_t (&pr)[2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = u0 + h;
                const int s = u / NBG;
                const int bb = u % NBG;
                const u32x4_t p = pb[u % D];
                // the pair bytes of the four B operands (any3: the fourth from the top bits)
                const u32x4_t pd = A3 ? u32x4_t{p[0], p[1], p[2], any3_top_pairs(p)} : p;
                // a chunk past K reads the zero zone instead of its table
                const uint32_t sv =
                    s1[bb >> 1] + (cbase + s < Kc ? 0u : Cfg::ZERO - (bb >> 1) * 65536u);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    if constexpr (I4) {
                        bw[h][s4] = u32x4_t{p[s4], 0u, 0u, 0u};   // decoded later
                    } else if constexpr (A2) {
                        // bytes 2*s4 and 2*s4+1: four weights each, one 64-bit read
                        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const int bi = 2 * s4 + t;
                            const u32x2_t q = lds_at<u32x2_t>(
                                smem, __builtin_amdgcn_perm(p[bi >> 2], sv,
                                                            0x0C020000u | ((4u + (bi & 3)) << 8)) +
                                          (bb & 1) * 128);
                            bw[h][s4][2 * t] = q[0];
                            bw[h][s4][2 * t + 1] = q[1];
                        }
                    } else {
#pragma unroll
                        for (int jb = 0; jb < 4; ++jb)
                            bw[h][s4][jb] = lds_at<uint32_t>(
                                smem, __builtin_amdgcn_perm(pd[s4], sv,
                                                            0x0C020000u | ((4u + jb) << 8)) +
                                          (bb & 1) * 128);
                    }
                }
                pr[h] = lds_at<uint32_t>(smem, ab_c[s] + bb * Cfg::AB_BLK);
            }
        };
        fetch(0, bwp[0], prp[0]);
#pragma unroll
        for (int u0 = 0; u0 < GS; u0 += 2) {
            // Issue priority alternates every two pairs.  Two waves share a
            // SIMD; at equal priority the older one is always preferred, runs
            // ahead, and the younger one then finishes alone.
            if ((u0 >> 2) & 1)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
            const int cur = (u0 >> 1) & 1;
            if (u0 + 2 < GS)
                fetch(u0 + 2, bwp[cur ^ 1], prp[cur ^ 1]);
            u32x4_t (&bw)[2][4] = bwp[cur];
            // x of the pair's chunk(s) from LDS (M <= 2); lanes of rows m >= M
            // read row M-1: those MFMA rows are never stored
            // (a pair spans two chunks when NBG is odd)
            constexpr int NX = NBG % 2 == 1 ? 2 : 1;
            u32x4_t xv[XSTREAM ? 1 : NX][4];
            if constexpr (!XSTREAM) {
#pragma unroll
                for (int h = 0; h < NX; ++h) {
                    const int c = cbase + (u0 + h) / NBG;
                    // a chunk past K reads the zeroed bytes behind x, never the
                    // next x row (its weights are zero, and 0 * inf is not)
                    const uint32_t xo =
                        c < Kc ? Cfg::XS + (static_cast<uint32_t>(j < M ? j : M - 1) * K +
                                            c * TILE_K + kq * 32) * 2
                               : Cfg::XS + ((xbytes + 15u) & ~15u) + kq * 64;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        xv[h][s4] = lds_at<u32x4_t>(smem, xo + s4 * 16);
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = u0 + h;
                const int s = u / NBG;
                const int bb = u % NBG;
                const bool live = gi * NBG + bb < nblk && cbase + s < Kc;
                const uint32_t pr = prp[cur][h] & (live ? 0xFFFFFFFFu : 0u);
                const float a = __builtin_ldexpf(bf16_to_f32(pr & 0xFFFFu), rsc[bb]);
                const float bt = bf16_to_f32(pr >> 16);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    bw[h][s4] = I4 ? deq_int4(bw[h][s4][0], a, bt) : deq_quad(bw[h][s4], a, bt);
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int s = (u0 + h) / NBG;
                    const int bb = (u0 + h) % NBG;
                    const u32x4_t& xa =
                        XSTREAM ? xq[s % DS][s4] : xv[XSTREAM || NX == 1 ? 0 : h][s4];
                    f32x4_t& ac = acc[bb][NBG == 1 ? h : 0];
                    ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, bw[h][s4]),
                        ac, 0, 0, 0);
                }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                issue(gi, u0 + h + D);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (ngroups > 0) {
        __syncthreads();
        reduce_store(ngroups - 1);
    }
}

// ---- k_gemm_kb: k-major for any K ------------------------------------------
//
// The k_gemm_km scheme for K > 4096: a workgroup owns row blocks r, r+Gs, ...
// and decodes NBG of them together; wave w owns chunks [w*C, (w+1)*C) with
// C = ceil(K/128 / 8), and walks them in steps of one chunk (the chunk's
// tile of every block of the group).  The loop body is unrolled over DS
// steps (the ring depth); a group's steps are padded to a multiple of DS
// with dead steps (out-of-range loads, and a uniform branch skips their
// decode).  x: with XL (M <= 2, one block per group, x small enough) x is copied
// to LDS in the prologue and each chunk's operands are read from there by
// the lanes of rows m < M; otherwise x travels in the ring, its operand
// loads for a chunk following the chunk's last tile.  alpha and beta of a
// whole group are staged in LDS by all threads, two 16-byte pieces per
// thread and tensor at most.
//
// LDS:
//   [0, TABS)  pair tables as in k_gemm_km (the partial sums reuse them)
//   AB         [NBG][GMAX][16 rows] (alpha | beta << 16) dwords
//   LUTS       [NBG][16 rows][16] f16, each row scaled by 2^-s
//   SCL        [NBG][16 rows] int: the row scale exponents s
//   XS         (XL) x as [M][K] bf16
constexpr int KB_XL_PIECES = 7;   // 16-byte pieces of x per thread (XL): 56 KB

template <int NBG, bool XL>
struct KbCfg {
    static_assert(!XL || NBG == 1, "x in LDS goes with one block per group");
    static constexpr int GMAX = NBG == 1 ? 512 : NBG == 2 ? 256 : NBG == 3 ? 144 : 112;
    static constexpr int TABS = ((NBG + 1) / 2) * 65536;
    static constexpr int ZERO = TABS;   // 256 zero bytes: the table reads of dead tiles
    static constexpr int AB_BLK = GMAX * 16 * 4;
    static constexpr int AB = ZERO + 256;
    static constexpr int LUTS = AB + NBG * AB_BLK;
    static constexpr int SCL = LUTS + NBG * 512;
    static constexpr int XS = SCL + NBG * 64;
    static constexpr int XMAX = XL ? KB_XL_PIECES * GT * 16 : 0;   // bytes of x in LDS
    static constexpr int LDS = XS + XMAX;
    // ring depth in chunks: x in the ring costs 16 VGPRs per chunk
    static constexpr int DS = XL ? 10 : (NBG == 1 ? 6 : NBG == 2 ? 4 : 2);
    static constexpr int D = DS * NBG;                             // ... in tiles
    static_assert(D % 2 == 0, "tiles are decoded in pairs");
    static_assert(LDS <= 160 * 1024, "LDS of one CU");
};

template <int MT, int NBG, bool XL, int FMT>
__global__ __launch_bounds__(GT) void k_gemm_kb(const GemmArgs args)
{
    constexpr bool I4 = FMT == FMT_INT4;
    constexpr bool A2 = FMT == FMT_ANY2;
    constexpr bool A3 = FMT == FMT_ANY3;
    constexpr uint32_t TB = tile_bytes(FMT);
    using Cfg = KbCfg<NBG, XL>;
    constexpr int DS = Cfg::DS;
    constexpr int D = Cfg::D;
    constexpr int NA = NBG == 1 ? 2 : 1;   // one block: two chains, added at the end
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int kq = lane >> 4;
    const int Kc = K / TILE_K;
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = K / g;
    const int Gs = gridDim.x;
    const int r = blockIdx.x;
    const int nblk = r < NB ? (NB - 1 - r) / Gs + 1 : 0;
    const int ngroups = (nblk + NBG - 1) / NBG;
    const int C = (Kc + GW - 1) / GW;        // chunks per wave
    const int CP = (C + DS - 1) / DS * DS;   // ... padded to whole bodies
    const int cbase = wave * C;
    const float inv_gc = 1.0f / static_cast<float>(g / TILE_K);   // chunk -> group

    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TB);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, static_cast<uint32_t>(N) * 32);
    // alpha/beta are read with 16-byte loads: the range is rounded up to 16 B
    // (the 16-byte granule holding a valid byte never leaves that byte's page
    // when the base is 16-byte aligned); the extra values only reach rows >= N.
    const uint32_t ab_range = (static_cast<uint32_t>(N) * G * 2 + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, ab_range);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, ab_range);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // ---- staging of a group.  Table rows: thread t < 32*NBG fetches piece
    // t % 32 of block t / 32.  alpha and beta: piece q = t + 512h (h < 2) is
    // piece q % 2G of block q / 2G.  Offsets carry the out-of-range bit
    // instead of a select.
    const int ab_per = 2 * G;
    int ab_blk[2], ab_pc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = tid + h * GT;
        ab_blk[h] = q / ab_per;
        ab_pc[h] = q - ab_blk[h] * ab_per;
    }
    auto stage_load = [&](int gi, u32x4_t& lq, u32x4_t (&aq)[2], u32x4_t (&bq)[2]) {
        {
            const int ib = tid >> 5;
            const int blk = gi * NBG + ib;
            const bool live = tid < 32 * NBG && blk < nblk;
            const uint32_t o = (static_cast<uint32_t>(r + blk * Gs) * 512 + (tid & 31) * 16) |
                               (static_cast<uint32_t>(!live) << 31);
            if constexpr (!I4)
                lq = load16(rl, o);
            else
                lq = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int blk = gi * NBG + ab_blk[h];
            const bool live = ab_blk[h] < NBG && blk < nblk;
            const uint32_t o =
                (static_cast<uint32_t>(r + blk * Gs) * (G * 32) + ab_pc[h] * 16) |
                (static_cast<uint32_t>(!live) << 31);
            aq[h] = load16(ra, o);
            bq[h] = load16(rb, o);
        }
    };
    auto stage_store = [&](const u32x4_t& lq, const u32x4_t (&aq)[2], const u32x4_t (&bq)[2]) {
        int sc = 0;
        u32x4_t lh = lq;
        if constexpr (!I4) {
            sc = lut_scale(lq);   // all lanes: pairs of lanes share a row
            lh = lut_to_f16(lq, sc);
        }
        if (!I4 && tid < 32 * NBG) {
            lds_at<u32x4_t>(smem, Cfg::LUTS + tid * 16) = lh;
            if ((tid & 1) == 0)
                lds_at<int>(smem, Cfg::SCL + (tid >> 1) * 4) = sc;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (ab_blk[h] < NBG)
                store_pairs(smem, Cfg::AB + ab_blk[h] * Cfg::AB_BLK, ab_pc[h], G, aq[h], bq[h]);
    };
    auto build = [&](int bb) {
        if constexpr (A2)
            build_table2<GW>(smem, Cfg::LUTS + bb * 512, (bb >> 1) * 65536 + (bb & 1) * 128, tid);
        else if constexpr (!I4)
            build_table<GW, A3>(smem, Cfg::LUTS + bb * 512, (bb >> 1) * 16384 + (bb & 1) * 32,
                                tid);
    };

    // ---- ring.  Tile u of a body whose first step is (group gc, padded step
    // sc) is chunk cbase + sc + u / NBG of block gc*NBG + u % NBG; past the
    // group's CP steps the sequence continues with the next group.
    u32x4_t pb[D];
    u32x4_t xq[XL ? 1 : DS][4];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * (TB / 64);
    const uint32_t x_lane = j < M ? static_cast<uint32_t>(j * K + kq * 32) * 2 : OOR;
    auto issue = [&](int gc, int sc, int uu) {
        int st = sc + uu / NBG;
        int gg = gc;
        if (st >= CP) {
            st -= CP;
            ++gg;
        }
        const int bb = uu % NBG;
        const int blk = gg * NBG + bb;
        const int c = cbase + st;
        const bool live = blk < nblk && st < C && c < Kc;
        const uint32_t uo =
            (static_cast<uint32_t>(r + blk * Gs) * static_cast<uint32_t>(Kc) + c) * TB |
            (static_cast<uint32_t>(!live) << 31);
        pb[uu % D] = A2   ? load8_nt(rp, off2(tile_lane, uo))
                     : A3 ? load12_nt(rp, off2(tile_lane, uo))
                          : load16_nt(rp, off2(tile_lane, uo));
        if (!XL && bb == NBG - 1) {
            const bool xl = gg < ngroups && st < C && c < Kc;
            const uint32_t xc =
                static_cast<uint32_t>(c) * TILE_K * 2 | (static_cast<uint32_t>(!xl) << 31);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                xq[XL ? 0 : (uu / NBG) % DS][s4] = load16(rx, off2(x_lane, xc) + s4 * 16);
        }
    };

    // ---- prologue (as in k_gemm_km); with XL, x goes to LDS first
    u32x4_t xc16[XL ? KB_XL_PIECES : 1];
    const uint32_t xbytes = static_cast<uint32_t>(M) * K * 2;
    if constexpr (XL) {
#pragma unroll
        for (int i = 0; i < KB_XL_PIECES; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * GT) * 16;
            xc16[i] = load16(rx, o < xbytes ? o : OOR);
        }
    }
    u32x4_t lq, aq[2], bq[2];
    stage_load(0, lq, aq, bq);
    constexpr int R0 = 2;
#pragma unroll
    for (int u = 0; u < R0; ++u)
        issue(0, 0, u);
    if (tid < 16)
        lds_at<u32x4_t>(smem, Cfg::ZERO + tid * 16) = u32x4_t{0u, 0u, 0u, 0u};
    stage_store(lq, aq, bq);
    if constexpr (XL) {
        // past x the region is zeroed (see k_gemm_km)
#pragma unroll
        for (int i = 0; i < KB_XL_PIECES; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * GT) * 16;
            lds_at<u32x4_t>(smem, Cfg::XS + o) = o < xbytes ? xc16[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();
    {
        constexpr int PER = (D - R0 + NBG - 1) / NBG;
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb) {
            build(bb);
#pragma unroll
            for (int u = R0 + bb * PER; u < R0 + (bb + 1) * PER && u < D; ++u)
                issue(0, 0, u);
        }
    }
    __syncthreads();

    // the lane's slot in a table entry (any2: 16 slots of 8 bytes)
    const uint32_t slot4 = A2 ? static_cast<uint32_t>(lane & 15) * 8 : static_cast<uint32_t>(lane & 31) * 4;
    const uint32_t s1[2] = {slot4, slot4 | 0x10000u};   // region 0 / region 1
    f32x4_t acc[NBG][NA];
#pragma unroll
    for (int bb = 0; bb < NBG; ++bb)
#pragma unroll
        for (int h = 0; h < NA; ++h)
            acc[bb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int rsc[NBG];
    auto load_scales = [&]() {
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb)
            rsc[bb] = I4 ? 0 : lds_at<int>(smem, Cfg::SCL + (bb * 16 + j) * 4);
    };
    load_scales();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);
    auto reduce_store = [&](int gi) {   // after a barrier: tables are free
#pragma unroll
        for (int bb = 0; bb < NBG; ++bb) {
            f32x4_t t = acc[bb][0];
            if constexpr (NA > 1)
                t += acc[bb][NA - 1];
            red[(bb * GW + wave) * 64 + lane] = t;
        }
        __syncthreads();
        const int blk = gi * NBG + wave;
        if (wave < NBG && blk < nblk)
            store_block<MT, GW>(red + wave * GW * 64, args.y, lane, M, N,
                                (r + blk * Gs) * TILE_ROWS);
    };

    u32x4_t lqn, aqn[2], bqn[2];
    const int total = ngroups * (CP / DS);
    int gc = 0, sc = 0;   // group and padded step of the body's first chunk
    for (int it = 0; it < total; ++it) {
        if (sc == 0) {
            if (gc > 0) {
                __syncthreads();
                reduce_store(gc - 1);
                stage_store(lqn, aqn, bqn);
                __syncthreads();
#pragma unroll
                for (int bb = 0; bb < NBG; ++bb)
                    build(bb);
                __syncthreads();
                load_scales();
#pragma unroll
                for (int bb = 0; bb < NBG; ++bb)
#pragma unroll
                    for (int h = 0; h < NA; ++h)
                        acc[bb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            stage_load(gc + 1, lqn, aqn, bqn);
        }
#pragma unroll
        for (int u0 = 0; u0 < D; u0 += 2) {
          // issue priority alternates every two pairs (see k_gemm_km)
          if ((u0 >> 2) & 1)
              __builtin_amdgcn_s_setprio(1);
          else
              __builtin_amdgcn_s_setprio(0);
          const int st0 = sc + u0 / NBG, st1 = sc + (u0 + 1) / NBG;
          const bool live0 = gc * NBG + u0 % NBG < nblk && st0 < C && cbase + st0 < Kc;
          const bool live1 = gc * NBG + (u0 + 1) % NBG < nblk && st1 < C && cbase + st1 < Kc;
          if (live0 || live1) {   // uniform: dead pairs (padding, absent blocks) are skipped
            u32x4_t bw[2][4];
            u32x4_t xv[XL ? 2 : 1][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = u0 + h;
                const int st = sc + u / NBG;
                const int bb = u % NBG;
                const u32x4_t p = pb[u];
                const u32x4_t pd = A3 ? u32x4_t{p[0], p[1], p[2], any3_top_pairs(p)} : p;
                const int c = cbase + st;
                const bool live = gc * NBG + bb < nblk && st < C && c < Kc;
                if constexpr (!I4) {
                    // a dead tile reads the zero zone instead of its table
                    const uint32_t sv =
                        s1[bb >> 1] + (live ? 0u : Cfg::ZERO - (bb >> 1) * 65536u);
                    if constexpr (A2) {
                        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
                        for (int bi = 0; bi < 8; ++bi) {   // four weights per byte
                            const u32x2_t q = lds_at<u32x2_t>(
                                smem, __builtin_amdgcn_perm(p[bi >> 2], sv,
                                                            0x0C020000u | ((4u + (bi & 3)) << 8)) +
                                          (bb & 1) * 128);
                            bw[h][bi >> 1][2 * (bi & 1)] = q[0];
                            bw[h][bi >> 1][2 * (bi & 1) + 1] = q[1];
                        }
                    } else {
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                            for (int jb = 0; jb < 4; ++jb)
                                bw[h][s4][jb] = lds_at<uint32_t>(
                                    smem, __builtin_amdgcn_perm(pd[s4], sv,
                                                                0x0C020000u | ((4u + jb) << 8)) +
                                              (bb & 1) * 128);
                    }
                }
                const int grp =
                    min(static_cast<int>((static_cast<float>(c) + 0.5f) * inv_gc), G - 1);
                const uint32_t pr =
                    lds_at<uint32_t>(smem, Cfg::AB + bb * Cfg::AB_BLK + (grp * 16 + j) * 4) &
                    (live ? 0xFFFFFFFFu : 0u);
                const float a = __builtin_ldexpf(bf16_to_f32(pr & 0xFFFFu), rsc[bb]);
                const float bt = bf16_to_f32(pr >> 16);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    bw[h][s4] = I4 ? deq_int4(p[s4], a, bt) : deq_quad(bw[h][s4], a, bt);
                if constexpr (XL) {
                    // the chunk's x in the operand layout; lanes of rows m >= M
                    // read row M-1 (those MFMA rows are never stored), so no
                    // branch splits the body
                    // a dead tile (w = 0) past K reads the last chunk: any finite x
                    const int cx = c < Kc ? c : Kc - 1;
                    const uint32_t xo =
                        Cfg::XS + (static_cast<uint32_t>(j < M ? j : M - 1) * K + cx * TILE_K +
                                   kq * 32) * 2;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        xv[h][s4] = lds_at<u32x4_t>(smem, xo + s4 * 16);
                }
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int u = u0 + h;
                    f32x4_t& ac = acc[u % NBG][NBG == 1 ? h : 0];
                    const u32x4_t& xa = XL ? xv[XL ? h : 0][s4] : xq[XL ? 0 : u / NBG][s4];
                    ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, bw[h][s4]),
                        ac, 0, 0, 0);
                }
          }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                issue(gc, sc, u0 + h + D);
        }
        sc += DS;
        if (sc == CP) {
            sc = 0;
            ++gc;
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (ngroups > 0) {
        __syncthreads();
        reduce_store(ngroups - 1);
    }
}

// ---- k_gemm_big: M > 16, a plain LDS-tiled MFMA GEMM over dequantised tiles --
//
// (Plain int4, any4_gemm_int4: no table pointer, the codes 0..15 are the values.)
// For batches past the decode sizes the product is compute-bound and each
// weight tile is used by many x rows, so the weights are dequantised once per
// workgroup into LDS and consumed from there.  A workgroup of 4 waves computes
// a BM x 64 block of y (BM rows of x, 64 rows of W = 4 row blocks): per chunk of
// 128 k, thread t dequantises its 16-byte slot of row block t / 64 (the slot
// of lane t % 64: row t % 16, k 32 * ((t % 64) / 16) .. + 31) exactly as
// any4_dequant does, into W's LDS tile, the threads copy x's BM x 128 tile
// (rows >= M read as zero), and after a barrier each wave multiplies its
// (BM/2) x 32 part with 16x16x32 bf16 MFMAs.  The global data of a chunk is
// fetched two chunks ahead (measured: 16% faster at M = 64 than one chunk
// ahead, 4-5% at M = 256 and 1024; a deeper ring costs occupancy).  A
// 128 x 128 variant with double-buffered LDS and one barrier per chunk was
// slower (346 against 305 us at M = 1024): one workgroup per CU leaves one
// wave per SIMD to hide the LDS latency.
//
// LDS: XS [BM][128 + 8] bf16, WS [64][128 + 8] bf16 (rows padded by 16 B so
// that the 16 rows of an operand read fall in different banks), LT [16][64][2]
// fp32 (the table rows of the workgroup's 64 weight rows, entry-major, each
// value twice so that a half wave's 32 lookups hit 32 banks; row-major, they
// cost about 7.7K cycles of bank conflicts per wave at M = 256).
constexpr int BIG_BN = 64;
constexpr int BIG_LD = TILE_K + 8;   // padded row length in bf16
constexpr int BIG_PF = 2;            // chunks of global data in flight per thread

template <int BM, int FMT, int BN = BIG_BN>
__global__ __launch_bounds__(256) void k_gemm_big(const GemmArgs args)
{
    constexpr bool A2 = FMT == FMT_ANY2;
    constexpr bool A3 = FMT == FMT_ANY3;
    constexpr uint32_t TB = tile_bytes(FMT);
    constexpr int MTW = BM / 32;   // 16-row m tiles per wave (the wave's BM/2 rows)
    constexpr int NTW = BN / 32;   // 16-row n tiles per wave (the wave's BN/2 rows)
    constexpr int SL = BN / 64;    // dequantisation slots per thread per chunk
    __shared__ __attribute__((aligned(16))) uint16_t xs[BM * BIG_LD];
    __shared__ __attribute__((aligned(16))) uint16_t ws[BN * BIG_LD];
    // table values as fp32, [entry][row][2 copies]: the 32 lanes of a half
    // wave (16 rows x two k quarters) read 32 different banks
    __shared__ float lt[16 * BN * 2];

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int Kc = K / TILE_K;
    const int G = K / g;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;

    // table rows of the 64 weight rows (rows >= N: zeros); no table (plain
    // int4): the codes themselves, 0..15
    for (int e = tid; e < BN * 16; e += 256) {
        const int n = n0 + e / 16;
        const float v = n >= N      ? 0.f
                        : args.lut ? bf16_to_f32(args.lut[static_cast<size_t>(n) * 16 + (e & 15)])
                                   : static_cast<float>(e & 15);
        lt[(e & 15) * BN * 2 + (e / 16) * 2] = v;
        lt[(e & 15) * BN * 2 + (e / 16) * 2 + 1] = v;
    }

    // this thread's dequantisation slots: row block wave + 4*sl of the
    // workgroup's BN/16, the lane's slot of its tile
    int wrow[SL], wn[SL], blk[SL];
    bool wlive[SL];
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
        const int tb = (tid >> 6) + 4 * sl;  // row block within the workgroup
        wrow[sl] = tb * 16 + (lane & 15);    // row within the BN
        wn[sl] = n0 + wrow[sl];
        blk[sl] = (n0 >> 4) + tb;            // global row block
        wlive[sl] = wn[sl] < N;
    }
    const int wk = (lane >> 4) * 32;         // k offset within the chunk

    f32x4_t acc[MTW][NTW];
#pragma unroll
    for (int a = 0; a < MTW; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
            acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int wm = (wave >> 1) * (BM / 2);   // the wave's rows within BM
    const int wc = (wave & 1) * (BN / 2);    // ... and columns within the BN
    const int j = lane & 15;
    const int kq = lane >> 4;

    // chunk c's global data, fetched BIG_PF chunks ahead into a register ring:
    // this thread's packed slot, its group's alpha and beta, and its x
    // pieces.  Bounds-checked buffer loads with the offset pushed out of range
    // (rows past N or M, chunks past K) instead of branches, so that the
    // compiler's wait counts follow the ring.
    constexpr int PF = BIG_PF;
    constexpr int XP = BM * 16 / 256;   // 16-byte x pieces per thread
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(args.packed, static_cast<uint32_t>((N + TILE_ROWS - 1) / TILE_ROWS) * Kc * TB);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, static_cast<uint32_t>(N) * G * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, static_cast<uint32_t>(N) * G * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);
    u32x4_t pk[PF][SL];
    uint32_t ab[PF][SL];
    u32x4_t xv[PF][XP];
    auto fetch = [&](int c, int sl) {
#pragma unroll
        for (int q = 0; q < SL; ++q) {
            const uint32_t dead = static_cast<uint32_t>(!wlive[q] || c >= Kc) << 31;
            const uint32_t po =
                ((static_cast<uint32_t>(blk[q]) * Kc + c) * TB + lane * (TB / 64)) | dead;
            if constexpr (A2) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rp, po, 0, 0);
                pk[sl][q] = u32x4_t{v[0], v[1], 0u, 0u};
            } else if constexpr (A3) {
                typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
                const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(rp, po, 0, 0);
                pk[sl][q] = u32x4_t{v[0], v[1], v[2], 0u};
            } else {
                pk[sl][q] = load16(rp, po);
            }
            const uint32_t ao = ((static_cast<uint32_t>(wn[q]) * G +
                                  static_cast<uint32_t>(c * TILE_K + wk) / g) * 2) |
                                dead;
            ab[sl][q] =
                static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(ra, ao, 0, 0)) |
                (static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rb, ao, 0, 0)) << 16);
        }
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int piece = tid + i * 256;
            const int m = m0 + (piece >> 4);
            const uint32_t xo =
                ((static_cast<uint32_t>(m) * K + c * TILE_K + (piece & 15) * 8) * 2) |
                (static_cast<uint32_t>(m >= M || c >= Kc) << 31);
            xv[sl][i] = load16(rx, xo);
        }
    };
#pragma unroll
    for (int sl = 0; sl < PF; ++sl)
        fetch(sl, sl);
    for (int c0 = 0; c0 < Kc; c0 += PF) {
#pragma unroll
        for (int sl = 0; sl < PF; ++sl) {
            const int c = c0 + sl;   // chunks past K (the last round) add zeros
            __syncthreads();   // the previous chunk's tiles are consumed (and lt is written)
            // weights: 32 per slot, exactly the any4_dequant values
#pragma unroll
            for (int q = 0; q < SL; ++q) {
                u32x4_t out[4] = {};
                if (wlive[q] && c < Kc) {
                    const float a = bf16_to_f32(ab[sl][q] & 0xFFFFu);
                    const float bt = bf16_to_f32(ab[sl][q] >> 16);
                    // entry i of this lane's row (its copy for the lane's half wave)
                    const float* Lr = lt + wrow[q] * 2 + ((lane >> 4) & 1);
                    auto L = [&](uint32_t i) { return Lr[i * (BN * 2)]; };
                    // bf16(a*l0 + b) | bf16(a*l1 + b) << 16 with one conversion
                    auto deq2 = [&](float l0, float l1) {
                        typedef float f2_t __attribute__((ext_vector_type(2)));
                        typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
                        const f2_t w = {fmaf(a, l0, bt), fmaf(a, l1, bt)};
                        return __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf2_t));
                    };
                    const u32x4_t p = pk[sl][q];
                    if constexpr (A2) {   // 8 bytes of four 2-bit codes: dwords 2i, 2i+1
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const uint32_t byte = (p[i >> 2] >> (8 * (i & 3))) & 0xFFu;
#pragma unroll
                            for (int t = 0; t < 2; ++t) {
                                const int d = 2 * i + t;
                                out[d >> 2][d & 3] =
                                    deq2(L((byte >> (4 * t)) & 3u), L((byte >> (4 * t + 2)) & 3u));
                            }
                        }
                    } else if constexpr (A3) {   // 16 pair indices: dwords 0-2, then the top bits
                        const uint32_t top = any3_top_pairs(p);
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const uint32_t P =
                                ((q < 12 ? p[q >> 2] : top) >> (8 * (q & 3))) & 0x3Fu;
                            out[q >> 2][q & 3] = deq2(L(P & 7u), L(P >> 3));
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const uint32_t byte = (p[q >> 2] >> (8 * (q & 3))) & 0xFFu;
                            out[q >> 2][q & 3] = deq2(L(byte & 15u), L(byte >> 4));
                        }
                    }
                }
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(ws + wrow[q] * BIG_LD + wk);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dst[q] = out[q];
            }
            // x: BM rows x 128 k
#pragma unroll
            for (int i = 0; i < XP; ++i) {
                const int piece = tid + i * 256;
                *reinterpret_cast<u32x4_t*>(xs + (piece >> 4) * BIG_LD + (piece & 15) * 8) =
                    xv[sl][i];
            }
            fetch(c + PF, sl);
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < TILE_K / 32; ++ks) {
                const int k = ks * 32 + kq * 8;
                u32x4_t bf[NTW];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    bf[nt] = *reinterpret_cast<const u32x4_t*>(ws + (wc + nt * 16 + j) * BIG_LD + k);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    const u32x4_t af =
                        *reinterpret_cast<const u32x4_t*>(xs + (wm + mt * 16 + j) * BIG_LD + k);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, bf[nt]),
                            acc[mt][nt], 0, 0, 0);
                }
            }
        }
    }
    // lane l holds y[m = 4 * (l / 16) + v][n = l % 16] of each 16 x 16 tile
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm + mt * 16 + kq * 4 + v;
                const int n = n0 + wc + nt * 16 + j;
                if (m < M && n < N)
                    args.y[static_cast<size_t>(m) * N + n] =
                        static_cast<uint16_t>(f32_to_bf16(acc[mt][nt][v]));
            }
}

// ---------------------------------------------------------------------------
// quantiser
// ---------------------------------------------------------------------------
// binary64 -> bf16 bits with a single rounding to nearest even: the value is
// first narrowed to binary32 with round-to-odd (truncate, then set the last
// bit if anything was dropped), which keeps enough information for the
// second rounding, binary32 -> bf16 to nearest even, to equal the direct one.
__device__ __forceinline__ uint32_t f64_to_bf16(double d)
{
    if (d != d)
        return 0x7FC0u;
    float f = __double2float_rz(d);
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (static_cast<double>(f) != d && (u & 0x7F800000u) != 0x7F800000u)
        u |= 1u;
    return f32_to_bf16(__builtin_bit_cast(float, u));
}

__device__ __forceinline__ double bf16_to_f64(uint32_t h)
{
    return static_cast<double>(bf16_to_f32(h));
}

// index of the nearest of the first Q table values (ties: the lower index)
__device__ __forceinline__ int nearest_q(double v, const double (&L)[16], int Q)
{
    int best = 0;
    double bd = fabs(v - L[0]);
#pragma unroll
    for (int q = 1; q < 16; ++q) {
        const double d = fabs(v - L[q]);
        if (q < Q && d < bd) {
            bd = d;
            best = q;
        }
    }
    return best;
}

// One thread per weight row, everything in binary64 and in the order below,
// so that the result is a deterministic function of the inputs (Q = 16 table
// values for any4, 8 for any3, 4 for any2):
//   1. per group of g weights: beta = bf16(min), alpha = bf16((max - min) / (Q - 1))
//   2. normalised weights ws = (w - beta) / alpha (0 where alpha = 0), their
//      importance wt = alpha * ex[k]
//   3. table L = 0, 1, .., Q-1; `iters` rounds of: every weight to its
//      nearest table value, then L[q] = sum(wt * ws) / sum(wt) over the
//      members of q in increasing k (products and sums rounded separately);
//      empty clusters keep their value
//   4. table stored in bf16 (entries from Q on: zero); every weight assigned
//      to the nearest stored value
// The per-thread sums live in LDS: [2][16][QT] doubles.
constexpr int QT = 64;   // threads (rows) per workgroup

__global__ __launch_bounds__(QT) void k_quantize(const float* __restrict__ W,
                                                 const float* __restrict__ ex,
                                                 uint8_t* __restrict__ idx,
                                                 uint16_t* __restrict__ lut,
                                                 uint16_t* __restrict__ alpha,
                                                 uint16_t* __restrict__ beta, int N, int K,
                                                 int g, int iters, int Q)
{
    __shared__ double sums[2][16][QT];
    const int t = threadIdx.x;
    const int n = blockIdx.x * QT + t;
    if (n >= N)
        return;   // no barrier follows: the sums are per thread
    const int G = K / g;
    const float* row = W + static_cast<size_t>(n) * K;
    uint16_t* an = alpha + static_cast<size_t>(n) * G;
    uint16_t* bn = beta + static_cast<size_t>(n) * G;

    for (int j = 0; j < G; ++j) {   // 1. group scale
        double lo = row[j * g], hi = lo;
        for (int k = j * g + 1; k < (j + 1) * g; ++k) {
            const double v = row[k];
            lo = v < lo ? v : lo;
            hi = v > hi ? v : hi;
        }
        bn[j] = static_cast<uint16_t>(f64_to_bf16(lo));
        an[j] = static_cast<uint16_t>(f64_to_bf16((hi - lo) / static_cast<double>(Q - 1)));
    }

    double L[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        L[q] = q < Q ? q : 0;
    for (int it = 0; it < iters; ++it) {   // 3. weighted k-means
#pragma unroll
        for (int q = 0; q < 16; ++q)
            sums[0][q][t] = sums[1][q][t] = 0.0;
        for (int j = 0; j < G; ++j) {
            const double al = bf16_to_f64(an[j]);
            const double be = bf16_to_f64(bn[j]);
            for (int k = j * g; k < (j + 1) * g; ++k) {
                const double ws = al != 0.0 ? (static_cast<double>(row[k]) - be) / al : 0.0;
                const double wt = __dmul_rn(al, static_cast<double>(ex[k]));
                const int q = nearest_q(ws, L, Q);
                sums[0][q][t] = __dadd_rn(sums[0][q][t], __dmul_rn(wt, ws));
                sums[1][q][t] = __dadd_rn(sums[1][q][t], wt);
            }
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (q < Q && sums[1][q][t] > 0.0)
                L[q] = sums[0][q][t] / sums[1][q][t];
    }

    double Lq[16];   // 4. the stored table and the final assignment
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t h = q < Q ? f64_to_bf16(L[q]) : 0u;
        lut[static_cast<size_t>(n) * 16 + q] = static_cast<uint16_t>(h);
        Lq[q] = bf16_to_f64(h);
    }
    uint8_t* in = idx + static_cast<size_t>(n) * K;
    for (int j = 0; j < G; ++j) {
        const double al = bf16_to_f64(an[j]);
        const double be = bf16_to_f64(bn[j]);
        for (int k = j * g; k < (j + 1) * g; ++k) {
            const double ws = al != 0.0 ? (static_cast<double>(row[k]) - be) / al : 0.0;
            in[k] = static_cast<uint8_t>(nearest_q(ws, Lq, Q));
        }
    }
}

// ---- k_quantize_w: the same quantiser, one wave per row ---------------------
// k_quantize's steps and roundings, spread over a wave's 64 lanes so that a
// layer's rows fill the chip (one thread per row leaves most CUs idle):
//   1. group scale: lane l folds groups l, l+64, ... exactly as k_quantize
//      (min and max in increasing k) and keeps the row's alpha | beta << 16
//      in LDS;
//   2-3. each k-means round walks the row in chunks of 64 consecutive k, one
//      per lane: every lane forms its weight's ws, wt = alpha * ex[k], its
//      nearest table value q and wt * ws (the E-step, in parallel) and leaves
//      (wt * ws, wt) in LDS; then lane q adds the chunk's members of cluster q
//      (a ballot per cluster names them) to its two sums in increasing k, so
//      each cluster's sums are rounded in k_quantize's order.  L[q] = sum /
//      weight for the non-empty clusters, broadcast from lane q;
//   4. the stored table, and the final assignment one weight per lane.
// A wave touches only its own LDS, so there is no barrier; rows with more
// than QW_MAX_G groups (not enough LDS for their alpha/beta) use k_quantize.
constexpr int QW_WAVES = 4;
constexpr int QW_MAX_G = 1024;

__global__ __launch_bounds__(64 * QW_WAVES) void k_quantize_w(const float* __restrict__ W,
                                                              const float* __restrict__ ex,
                                                              uint8_t* __restrict__ idx,
                                                              uint16_t* __restrict__ lut,
                                                              uint16_t* __restrict__ alpha,
                                                              uint16_t* __restrict__ beta, int N,
                                                              int K, int g, int iters, int Q)
{
    __shared__ uint32_t ab_s[QW_WAVES][QW_MAX_G];   // alpha | beta << 16 per group
    __shared__ double pw_s[QW_WAVES][2][64];        // a chunk's (wt * ws, wt) per lane
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = blockIdx.x * QW_WAVES + wv;
    if (n >= N)
        return;   // whole waves: nothing below waits for another wave
    const int G = K / g;
    const float* row = W + static_cast<size_t>(n) * K;
    uint32_t* ab = ab_s[wv];
    double* pw0 = pw_s[wv][0];
    double* pw1 = pw_s[wv][1];

    for (int j = lane; j < G; j += 64) {   // 1. group scale
        double lo = row[j * g], hi = lo;
        for (int k = j * g + 1; k < (j + 1) * g; ++k) {
            const double v = row[k];
            lo = v < lo ? v : lo;
            hi = v > hi ? v : hi;
        }
        const uint32_t b = f64_to_bf16(lo);
        const uint32_t a = f64_to_bf16((hi - lo) / static_cast<double>(Q - 1));
        beta[static_cast<size_t>(n) * G + j] = static_cast<uint16_t>(b);
        alpha[static_cast<size_t>(n) * G + j] = static_cast<uint16_t>(a);
        ab[j] = a | (b << 16);
    }
    __builtin_amdgcn_wave_barrier();

    // ws and wt of weight k (its group's alpha and beta from LDS)
    auto weight = [&](int k, double& ws, double& al) {
        const uint32_t p = ab[k / g];
        al = bf16_to_f64(p & 0xFFFFu);
        const double be = bf16_to_f64(p >> 16);
        ws = al != 0.0 ? (static_cast<double>(row[k]) - be) / al : 0.0;
    };

    double L[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        L[q] = q < Q ? q : 0;
    const int nch = (K + 63) / 64;
    for (int it = 0; it < iters; ++it) {   // 3. weighted k-means
        double S = 0.0, T = 0.0;           // lane q: the sums of cluster q
        for (int c = 0; c < nch; ++c) {
            const int k = c * 64 + lane;
            int q = 16;   // no cluster: a lane past K
            double pr = 0.0, wt = 0.0;
            if (k < K) {
                double ws, al;
                weight(k, ws, al);
                wt = __dmul_rn(al, static_cast<double>(ex[k]));
                q = nearest_q(ws, L, Q);
                pr = __dmul_rn(wt, ws);
            }
            pw0[lane] = pr;
            pw1[lane] = wt;
            uint64_t mine = 0;   // lane q: the lanes of the chunk in cluster q
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) {
                if (qq < Q) {
                    const uint64_t m = __builtin_amdgcn_ballot_w64(q == qq);
                    mine = lane == qq ? m : mine;
                }
            }
            __builtin_amdgcn_wave_barrier();
            while (mine) {   // in increasing k
                const int i = __builtin_ctzll(mine);
                mine &= mine - 1;
                S = __dadd_rn(S, pw0[i]);
                T = __dadd_rn(T, pw1[i]);
            }
            __builtin_amdgcn_wave_barrier();   // reads done before the next chunk's writes
        }
        const bool upd = lane < Q && T > 0.0;
        const double cand = upd ? S / T : 0.0;
        const uint64_t um = __builtin_amdgcn_ballot_w64(upd);
        const uint64_t cb = __builtin_bit_cast(uint64_t, cand);
        const uint32_t clo = static_cast<uint32_t>(cb), chi = static_cast<uint32_t>(cb >> 32);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if ((um >> q) & 1u) {
                // readlane returns int: widen through uint32_t, not with sign
                const uint32_t vlo = static_cast<uint32_t>(__builtin_amdgcn_readlane(clo, q));
                const uint32_t vhi = static_cast<uint32_t>(__builtin_amdgcn_readlane(chi, q));
                const uint64_t v = static_cast<uint64_t>(vlo) | (static_cast<uint64_t>(vhi) << 32);
                L[q] = __builtin_bit_cast(double, v);
            }
        }
    }

    double Lq[16];   // 4. the stored table and the final assignment
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t h = q < Q ? f64_to_bf16(L[q]) : 0u;
        if (lane == q)
            lut[static_cast<size_t>(n) * 16 + q] = static_cast<uint16_t>(h);
        Lq[q] = bf16_to_f64(h);
    }
    uint8_t* in = idx + static_cast<size_t>(n) * K;
    for (int k = lane; k < K; k += 64) {
        double ws, al;
        weight(k, ws, al);
        in[k] = static_cast<uint8_t>(nearest_q(ws, Lq, Q));
    }
}

// ---- k_read_probe: the streaming-read ceiling --------------------------------
// Reads a buffer once with the GEMM's loads (16 bytes per lane, non-temporal,
// a wave's 64 lanes on 1 KB contiguous) and writes one word (so the loads are
// not dead).  It measures what the memory system gives a kernel of this size
// and shape.  Shape: one workgroup of 16 waves per CU, each wave issuing all
// of its DEPTH loads at once, DEPTH = ceil(tiles / 4096) up to 16 (the best of
// a sweep over waves per workgroup, workgroups, loads per wave, ring or
// all-at-once issue and the non-temporal hint: on 29.4 MB, 16 x 7 over 256
// workgroups read in 5.45 us, against 5.55 us for 8 x 16 over 224 and 6.0 us
// without the hint).
constexpr int PROBE_WAVES = 16;
constexpr int PROBE_MAX_DEPTH = 16;

template <int DEPTH>
__global__ __launch_bounds__(64 * PROBE_WAVES) void k_read_probe(const uint8_t* __restrict__ p,
                                                                 uint32_t tiles,
                                                                 uint32_t* __restrict__ out)
{
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p, tiles * 1024u);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wid = blockIdx.x * PROBE_WAVES + (threadIdx.x >> 6);   // global wave
    const uint32_t nw = gridDim.x * PROBE_WAVES;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint32_t t0 = wid * DEPTH; t0 < tiles; t0 += nw * DEPTH) {
        u32x4_t v[DEPTH];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)   // past the end: out of range, reads zero
            v[i] = load16_nt(rs, (t0 + i) * 1024u + lane * 16u);
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)
            acc ^= v[i];
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u)
        out[0] = 1u;
}

// s_setprio for a priority known once the loop is unrolled (the builtin takes
// an immediate; the branches fold away)
__device__ __forceinline__ void st_prio(int p)
{
    if (p >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (p == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (p == 1)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// ---- k_gemm_st: the whole ring in flight from the first instruction --------
//
// The decode kernel for M <= 16.  A workgroup of NW waves (NW = blockDim/64,
// at most 16, chosen by the host) owns row blocks r, r+Gs, r+2Gs, ... and
// decodes them NBG at a time (a group); wave w owns chunks [w*cw, (w+1)*cw)
// of K (cw a multiple of R, chosen by the host) and walks them R at a time
// (a body), each step decoding that chunk's tile of every block of the
// group against the same x operands.
//
// A streaming read of this size only reaches HBM's bandwidth when every wave
// has its loads in flight from the start (MI355X, 29.4 MB in one launch:
// 5.45-5.5 us with all loads issued at once, 6.0-6.2 us with an 8-deep ring
// refilled as tiles are consumed).  So the ring holds a whole body (R*NBG
// tiles); for the decode shapes that is every tile the wave reads, and it
// is issued in the prologue right behind the small staging loads (table
// rows, alpha/beta, x for XL).  The staging data lands in LDS as soon as it
// arrives and the NBG pair tables are built with 16-byte writes while the
// tiles are still on their way.
//
// Decode, dequantisation and x operands as in k_gemm_km (pair tables of 32
// slots, each weight formed as bf16(fp32(alpha*L + beta)) from the row's
// 2^-s scaled f16 table values).  A dead tile (a block past the workgroup's
// last, a chunk past K) reads the 256 zero bytes at ZERO instead of its
// table, with alpha = beta = 0.
//
// LDS (byte offsets from st_layout):
//   [0, ZERO)  pair tables: table b in 64 KB region b/2, half b%2, entry e at
//              e*256 + (b%2)*128 + slot*4; the partial sums reuse it
//   ZERO       256 zero bytes (64 KB aligned: the table reads of dead tiles)
//   AB         [NBG][GS][16 rows] (alpha | beta << 16) dwords: the GS groups
//              from gbase on that the workgroup's chunks touch
//   LUTS       [NBG][4 row quads][16 entries][4 rows] f16, each row scaled by 2^-s
//   SCL        [NBG][16 rows] int: the row scale exponents s
//   XS, XZ     (XL) x as [M][K] bf16, then 256 zero bytes (x of dead chunks)
struct StLayout {
    uint32_t zero, ab, luts, scl, xs, xz, total;
};

// GS: the groups of alpha/beta staged per block (all K/g without a split of
// K, else those of one split's chunks)
__host__ __device__ inline StLayout st_layout(int nbg, int GS, int M, int K, bool xl)
{
    StLayout L;
    L.zero = static_cast<uint32_t>((nbg + 1) / 2) * 65536u;
    L.ab = L.zero + 256;
    L.luts = L.ab + static_cast<uint32_t>(nbg) * GS * 64;
    L.scl = L.luts + nbg * 512;
    L.xs = L.scl + nbg * 64;
    L.xz = L.xs + (xl ? ((static_cast<uint32_t>(M) * K * 2 + 15u) & ~15u) : 0u);
    L.total = L.xz + (xl ? 256u : 0u);
    return L;
}

constexpr int ST_MAX_WAVES = 16;
#ifndef ANY4_ST_W16_MAX_M
#define ANY4_ST_W16_MAX_M 32
#endif
constexpr int ST_W16_MAX_M = ANY4_ST_W16_MAX_M;   // 16 waves per CU up to this many x rows
constexpr int ST_LDS = 160 * 1024;   // one workgroup per CU: all of its LDS
constexpr int ST_XP = 4;   // 16-byte pieces of x per thread (XL)

struct StArgs {
    GemmArgs a;
    int splits;    // K is split over this many workgroups (partial sums in a.ws), at most 4
    int gstage;    // alpha/beta groups staged per block (GS)
    int cw;        // chunks per wave (a multiple of R)
    StLayout L;
    unsigned long long* ts;   // per-wave timestamps (probe builds only), or null
    // Launch constants the host works out, so that no integer division runs
    // between a wave's start and its first loads: K/g, g/128, workgroups per
    // split, chunks per split, the most row blocks a workgroup owns, the first
    // staged group of each split, and 1/(2 K/g), 1/(K/g) for small quotients
    int G, gc, Gs, KcS, nbmax;
    int gbase[4];
    float inv_abper, inv_G;
};

template <int MT, int NBG, int R, bool XL, bool MG, int LB, int PRE, int D, int FMT, bool VD = false>
__global__ __launch_bounds__(LB) void k_gemm_st(const StArgs sa)
{
    static_assert(!VD || (MT == 1 && XL), "the VALU dot path is the M = 1 product with x in LDS");
    static_assert(MT <= 16 || (MT % 16 == 0 && !XL && !VD), "wide batches: 16-row slices of x in the ring");
    // M > 16: MS slices of 16 x rows, each with its own MFMA chains against the
    // same decoded weights, so the weights are read once for all of them
    constexpr int MS = MT > 16 ? MT / 16 : 1;
    constexpr int MTS = MT > 16 ? 16 : MT;   // rows per slice
    constexpr bool I4 = FMT == FMT_INT4;
    constexpr bool A2 = FMT == FMT_ANY2;
    constexpr bool A3 = FMT == FMT_ANY3;
    constexpr uint32_t TB = tile_bytes(FMT);
    constexpr int TPW = R * NBG;   // tiles in a body
    static_assert(TPW % D == 0, "the ring depth divides a body");
    static_assert(XL || TPW - D >= NBG - 1, "x of a step is not overwritten before its step");
    constexpr bool XSTREAM = !XL;
    // static (not dynamic) LDS: its base is the constant 0, so table addresses
    // need no add
    __shared__ __attribute__((aligned(16))) uint8_t smem[ST_LDS];
    const GemmArgs& args = sa.a;
    const StLayout L = sa.L;

    const int M = args.M, N = args.N, K = args.K, g = args.g;
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NW = NT >> 6;
    const int j = lane & 15;
    const int kq = lane >> 4;
    const int Kc = K >> 7;   // K / TILE_K
    const int NB = (N + TILE_ROWS - 1) / TILE_ROWS;
    const int G = sa.G;
    const int gc = sa.gc;   // chunks per group
    (void)g;
    // with splits S (at most 4), workgroup r' = split * Gs + r takes chunks
    // [split*KcS, (split+1)*KcS) of the same row blocks as workgroup r
    const int S = sa.splits;
    const int Gs = sa.Gs;
    const int bx = blockIdx.x;
    const int split = (bx >= Gs) + (bx >= 2 * Gs) + (bx >= 3 * Gs);
    const int r = bx - split * Gs;
    const int KcS = sa.KcS;
    const int kend = min((split + 1) * KcS, Kc);   // chunks from kend on are dead
    // row blocks r, r+Gs, ... below NB: nbmax of them, or one fewer (r < Gs <= NB)
    const int nblk = sa.nbmax - 1 + (r + (sa.nbmax - 1) * Gs < NB ? 1 : 0);
    const int ngroups = MG ? (nblk + NBG - 1) / NBG : 1;
    const int cw = sa.cw;
    const int bpg = cw / R;        // bodies per group
    const int c0 = split * KcS + wave * cw;
    const int GS = sa.gstage;
    const int gbase = sa.gbase[split];   // first staged group
#ifdef ANY4_PROBE_TS
    unsigned long long* ts = sa.ts ? sa.ts + (static_cast<size_t>(r) * NW + wave) * 8 : nullptr;
    auto stamp = [&](int i) {
        if (ts && lane == 0)
            ts[i] = __builtin_amdgcn_s_memtime();
    };
#else
    auto stamp = [](int) {};
#endif
    stamp(0);

    const __amdgpu_buffer_rsrc_t rp = make_rsrc(args.packed, static_cast<uint32_t>(NB) * Kc * TB);
    // plain int4 has no table (its pointer may be null): nothing is read through rl
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(args.lut, I4 ? 0u : static_cast<uint32_t>(N) * 32);
    const uint32_t ab_range = (static_cast<uint32_t>(N) * G * 2 + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.alpha, ab_range);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(args.beta, ab_range);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x, static_cast<uint32_t>(M) * K * 2);

    // ---- staging of group gi.  Table rows: thread t < 32*NBG fetches 16 B
    // (8 entries of row (t%32)/2) of block t/32.  alpha/beta: item q = t + h*NT
    // (h < 2) is piece q % 2G of block q / 2G, 16 B of each tensor.
    // The prologue's per-lane arithmetic runs four waves to a SIMD before the
    // first loads go out, so waves with no live item skip it (uniform tests).
    const int ab_per = 2 * G;
    int ab_blk[2], ab_pc[2];
    bool ab_wave[2];   // the wave holds live alpha/beta items in round h
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ab_wave[h] = wave * 64 + h * NT < NBG * ab_per;
        const int q = tid + h * NT;
        ab_blk[h] = ab_wave[h] ? small_div(q, sa.inv_abper) : NBG;   // q < 2048
        ab_pc[h] = q - ab_blk[h] * ab_per;
    }
    // Early build (one group, pair tables, a build item per thread): the
    // lanes of a wave build items of one 64 KB table region (blocks 2p and
    // 2p+1, NBG even) or of one block (NBG odd), so each wave loads those
    // blocks' table rows itself (lanes 0-31 block 2p, 32-63 block 2p+1, or
    // lanes 0-31 the one block), stages them and builds its items without
    // waiting for the other waves; the waves of a block store identical
    // staging values.  Otherwise the first 32*NBG threads stage every
    // block's rows and the workgroup meets at a barrier before the build.
    constexpr bool EBC = !MG && !I4 && !A2;
    constexpr bool RM = NBG % 2 == 0;   // region-major build items
    const bool eb = EBC && NT >= NBG * 256;
    const bool lut_lane = eb ? tid < NBG * 256 && (RM || lane < 32) : tid < 32 * NBG;
    // block of the lane's staged rows: the wave's first (uniform), plus one
    // for lanes 32-63 where a wave stages two blocks
    const int lut_wb = eb ? (RM ? 2 * (wave >> 3) : wave >> 2) : 2 * wave;
    const int lut_hb = (!eb || RM) && lane >= 32 ? 1 : 0;
    const int lut_blk = lut_wb + lut_hb;
    auto stage_load = [&](int gi, u32x4_t& lq, u32x4_t (&aq)[2], u32x4_t (&bq)[2]) {
        {
            const int blk = gi * NBG + lut_blk;
            const bool live = lut_lane && blk < nblk;
            const uint32_t base = static_cast<uint32_t>(r + (gi * NBG + lut_wb) * Gs) * 512;   // uniform
            const uint32_t o = (base + (lut_hb ? static_cast<uint32_t>(Gs) * 512 : 0u) + (tid & 31) * 16) |
                               (static_cast<uint32_t>(!live) << 31);
            if constexpr (I4)
                lq = u32x4_t{0u, 0u, 0u, 0u};
            else
                lq = load16(rl, o);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            aq[h] = bq[h] = u32x4_t{0u, 0u, 0u, 0u};
            if (!ab_wave[h])
                break;   // uniform; the later rounds hold no live item either
            const int blk = gi * NBG + ab_blk[h];
            // the piece's 8 values are groups g0..g0+7 (mod G) of its rows:
            // loaded only if one of them is staged
            bool need = true;
            if (G > GS) {
                const int g0 = 8 * ab_pc[h] - G * small_div(8 * ab_pc[h], sa.inv_G);   // (8 pc) mod G
                need = (g0 + 7 >= gbase && g0 < gbase + GS) || (g0 + 7 >= G && (g0 + 7 - G) >= gbase);
            }
            const bool live = ab_blk[h] < NBG && blk < nblk && need;
            const uint32_t o = (static_cast<uint32_t>(r + blk * Gs) * (G * 32) + ab_pc[h] * 16) |
                               (static_cast<uint32_t>(!live) << 31);
            aq[h] = load16(ra, o);
            bq[h] = load16(rb, o);
        }
    };
    auto stage_store = [&](const u32x4_t& lq, const u32x4_t (&aq)[2], const u32x4_t (&bq)[2]) {
        const int sc = I4 ? 0 : lut_scale(lq);   // all lanes: lanes 2i, 2i+1 hold one row
        const u32x4_t lh = I4 ? lq : lut_to_f16(lq, sc);
        if (lut_lane) {
            // by row quad, entry, row: a build thread reads one entry of four
            // rows with one 8-byte read, eight entries with two 16-byte reads
            const int row = (tid & 31) >> 1;
            const uint32_t base = L.luts + lut_blk * 512 + (row >> 2) * 128 + (row & 3) * 2;
            const int e0 = (tid & 1) * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lds_at<uint16_t>(smem, base + (e0 + i) * 8) =
                    static_cast<uint16_t>(lh[i >> 1] >> (16 * (i & 1)));
            if ((tid & 1) == 0)
                lds_at<int>(smem, L.scl + (lut_blk * 16 + row) * 4) = sc;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (ab_wave[h] && ab_blk[h] < NBG)
                store_pairs_range(smem, L.ab + ab_blk[h] * GS * 64, ab_pc[h], G, sa.inv_G, gbase, GS, aq[h],
                                  bq[h]);
    };
    // Pair tables of the group with 16-byte writes.  Item (block b, half h,
    // hi, slot quad q) writes slots 4q..4q+3 (rows 4(q%4)..+3) of the entries
    // hi<<4 | lo, lo = 8h..8h+7, and the table values come from three LDS
    // reads.  Items are numbered it = b<<8 | h<<7 | hi<<3 | q (block-major:
    // the 8 lanes of one entry write its 128 contiguous bytes) or, region-
    // major, it = p<<9 | h<<8 | hi<<4 | (b&1)<<3 | q with p = b>>1 (the 16
    // lanes of one entry write both tables of the region: 256 contiguous
    // bytes, so one 16-byte write of a wave covers every LDS bank).
    auto build_item = [&](int b, int h, int hi, int q, auto&& hook) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const uint32_t src = L.luts + b * 512 + (q & 3) * 128;
        // any4: entry hi<<4 | lo is (L[lo], L[hi]).  any3: the byte's low 6
        // bits are two 3-bit codes and bits 6-7 pick one of four identical
        // copies, so entry e is (L[e & 7], L[(e >> 3) & 7]): for lo = 8h + i
        // that is (L[i], L[(2hi + h) & 7]).
        const uint32_t bsrc = A3 ? ((2 * hi + h) & 7) * 8 : hi * 8;
        const uint32_t asrc = A3 ? 0u : h * 64;
        const u32x2_t B = lds_at<u32x2_t>(smem, src + bsrc);         // second value, 4 rows
        const u32x4_t Q0 = lds_at<u32x4_t>(smem, src + asrc);        // first values of lo, lo+1
        const u32x4_t Q1 = lds_at<u32x4_t>(smem, src + asrc + 16);   // lo+2, lo+3
        const u32x4_t Q2 = lds_at<u32x4_t>(smem, src + asrc + 32);
        const u32x4_t Q3 = lds_at<u32x4_t>(smem, src + asrc + 48);
        const uint32_t Aw[16] = {Q0[0], Q0[1], Q0[2], Q0[3], Q1[0], Q1[1], Q1[2], Q1[3],
                                 Q2[0], Q2[1], Q2[2], Q2[3], Q3[0], Q3[1], Q3[2], Q3[3]};
        const uint32_t dst = (b >> 1) * 65536 + (b & 1) * 128 + (hi * 16 + h * 8) * 256 + q * 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a0 = Aw[2 * i], a1 = Aw[2 * i + 1];
            const u32x4_t v = {__builtin_amdgcn_perm(B[0], a0, 0x05040100u),
                               __builtin_amdgcn_perm(B[0], a0, 0x07060302u),
                               __builtin_amdgcn_perm(B[1], a1, 0x05040100u),
                               __builtin_amdgcn_perm(B[1], a1, 0x07060302u)};
            lds_at<u32x4_t>(smem, dst + i * 256) = v;
            hook(i);
        }
    };
    // any2: quad tables.  Entry e (a byte of four 2-bit codes c_s = (e >> 2s) & 3)
    // holds, per row, (L[c0] | L[c1] << 16, L[c2] | L[c3] << 16); 16 slots of
    // 8 bytes (slot = row), entry e at e*256 (+128 for the second table of a
    // 64 KB region).  Item it = (block, entry, slot pair q) writes rows 2q, 2q+1.
    auto build_item2 = [&](int it) {
        const int q = it & 7;
        const int e = (it >> 3) & 255;
        const int b = it >> 11;
        const uint32_t src = L.luts + b * 512 + (q >> 1) * 128 + (q & 1) * 4;
        uint32_t c[4];   // (L[c_s] of row 2q, of row 2q+1)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            c[t] = lds_at<uint32_t>(smem, src + ((e >> (2 * t)) & 3) * 8);
        const u32x4_t v = {__builtin_amdgcn_perm(c[1], c[0], 0x05040100u),
                           __builtin_amdgcn_perm(c[3], c[2], 0x05040100u),
                           __builtin_amdgcn_perm(c[1], c[0], 0x07060302u),
                           __builtin_amdgcn_perm(c[3], c[2], 0x07060302u)};
        lds_at<u32x4_t>(smem, (b >> 1) * 65536 + (b & 1) * 128 + e * 256 + q * 16) = v;
    };
    auto build = [&]() {
        if constexpr (A2) {
            for (int it = tid; it < NBG * 2048; it += NT)
                build_item2(it);
        } else if constexpr (!I4) {
            for (int it = tid; it < NBG * 256; it += NT)
                build_item(it >> 8, (it >> 7) & 1, (it >> 3) & 15, it & 7, [](int) {});
        }
    };

    // ---- ring.  Tile u of body k: step s = u / NBG (chunk c0 + (k % bpg)*R + s)
    // of block (k / bpg)*NBG + u % NBG; it sits in ring slot u % D (D divides
    // a body).  x (XSTREAM): a step's operands are loaded with its first tile.
    u32x4_t pb[D];
    u32x4_t xq[XSTREAM ? R : 1][MS][4];
    const uint32_t tile_lane = static_cast<uint32_t>(lane) * (TB / 64);
    uint32_t x_lane[MS];   // x row j + 16*ms of the lane's k quarter, or out of range
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
        x_lane[ms] = j + 16 * ms < M ? static_cast<uint32_t>((j + 16 * ms) * K + kq * 32) * 2 : OOR;
    auto issue = [&](int k, int u) {
        const int gi = k / bpg;
        const int s = (k - gi * bpg) * R + u / NBG;
        const int blk = gi * NBG + u % NBG;
        const int c = c0 + s;
        const bool live = gi < ngroups && blk < nblk && c < kend;
        const uint32_t uo = (static_cast<uint32_t>(r + blk * Gs) * static_cast<uint32_t>(Kc) + c) * TB |
                            (static_cast<uint32_t>(!live) << 31);
        pb[u % D] = A2   ? load8_nt(rp, off2(tile_lane, uo))
                    : A3 ? load12_nt(rp, off2(tile_lane, uo))
                         : load16_nt(rp, off2(tile_lane, uo));
        if constexpr (XSTREAM) {
            if (u % NBG == 0) {
                const bool xl = gi < ngroups && c < kend;
                const uint32_t xc = static_cast<uint32_t>(c) * TILE_K * 2 | (static_cast<uint32_t>(!xl) << 31);
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        xq[u / NBG][ms][s4] = load16(rx, off2(x_lane[ms], xc) + s4 * 16);
            }
        }
    };
    // the tile D places after tile u of body k
    auto issue_next = [&](int k, int u) {
        if (u + D < TPW)
            issue(k, u + D);
        else
            issue(k + 1, u + D - TPW);
    };

    // ---- prologue: staging loads, x (XL), the first PRE ring tiles; the rest
    // of the ring once the staging data is in (requested behind the whole
    // ring, it would queue behind every tile of the chip)
    u32x4_t lq, aq[2], bq[2];
    stage_load(0, lq, aq, bq);
    u32x4_t xc16[XL ? ST_XP : 1];
    const uint32_t xbytes = static_cast<uint32_t>(M) * K * 2;
    // the waves past x load nothing (uniform test)
    if constexpr (XL) {
#pragma unroll
        for (int i = 0; i < ST_XP; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * NT) * 16;
            xc16[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (static_cast<uint32_t>(wave * 64 + i * NT) * 16 < xbytes)
                xc16[i] = load16(rx, o < xbytes ? o : OOR);
        }
    }
#pragma unroll
    for (int u = 0; u < (PRE < D ? PRE : D); ++u)
        issue(0, u);
    stamp(1);
    if (tid < 16)
        lds_at<u32x4_t>(smem, L.zero + tid * 16) = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (XL) {
        if (tid < 16)
            lds_at<u32x4_t>(smem, L.xz + tid * 16) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < ST_XP; ++i) {
            const uint32_t o = static_cast<uint32_t>(tid + i * NT) * 16;
            if (o < xbytes)
                lds_at<u32x4_t>(smem, L.xs + o) = xc16[i];
        }
    }
    stage_store(lq, aq, bq);
    stamp(2);
    if (eb)
        asm volatile("" ::: "memory");   // the wave reads back its own staging writes (in order)
    else
        __syncthreads();
    stamp(3);
    // the tables' 16-byte writes and the rest of the ring's loads, interleaved,
    // so that neither the LDS nor the texture unit waits for the other
    if (!I4 && !A2 && NT >= NBG * 256) {
        if (tid < NBG * 256) {   // uniform: NBG * 256 is a multiple of 64
            const bool rm = eb && RM;
            build_item(rm ? 2 * (tid >> 9) + ((tid >> 3) & 1) : tid >> 8,
                       rm ? (tid >> 8) & 1 : (tid >> 7) & 1, rm ? (tid >> 4) & 15 : (tid >> 3) & 15,
                       tid & 7, [&](int i) {
                           if (PRE + i < D)
                               issue(0, PRE + i);
                       });
#pragma unroll
            for (int u = PRE + 8; u < D; ++u)
                issue(0, u);
        } else {
#pragma unroll
            for (int u = PRE; u < D; ++u)
                issue(0, u);
        }
    } else {
#pragma unroll
        for (int u = PRE; u < D; ++u)
            issue(0, u);
        build();
    }
    __syncthreads();
    stamp(4);

    // the lane's slot in a table entry (any2: 16 slots of 8 bytes)
    const uint32_t slot4 = A2 ? static_cast<uint32_t>(lane & 15) * 8 : static_cast<uint32_t>(lane & 31) * 4;
    f32x4_t acc[NBG][MS];
#pragma unroll
    for (int b = 0; b < NBG; ++b)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
            acc[b][ms] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float dacc[VD ? NBG : 1];   // VD: the lane's partial dot product per block
#pragma unroll
    for (int b = 0; b < (VD ? NBG : 1); ++b)
        dacc[b] = 0.f;
    int rsc[NBG];
    auto load_scales = [&]() {
#pragma unroll
        for (int b = 0; b < NBG; ++b)
            rsc[b] = I4 ? 0 : lds_at<int>(smem, L.scl + (b * 16 + j) * 4);
    };
    load_scales();
    const int jr = j < M ? j : M - 1;

    u32x4_t lqn, aqn[2], bqn[2];
    const int total = ngroups * bpg;
    for (int k = 0; k < total; ++k) {
        const int gi = k / bpg;
        const int kb = k - gi * bpg;
        if constexpr (MG) {
            if (kb == 0)
                stage_load(gi + 1, lqn, aqn, bqn);
        }
#pragma unroll
        for (int s = 0; s < R; ++s) {
            const int c = c0 + kb * R + s;
            const int grp = min(c / gc, G - 1);
            u32x4_t xv[4];
            if constexpr (XL) {
                const uint32_t xo = c < kend ? L.xs + (static_cast<uint32_t>(jr) * K + c * TILE_K + kq * 32) * 2
                                             : L.xz + kq * 64;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    xv[s4] = lds_at<u32x4_t>(smem, xo + s4 * 16);
            }
#pragma unroll
            for (int b = 0; b < NBG; ++b) {
                const int u = s * NBG + b;
                // The loop is VALU-bound and at equal priority the oldest wave
                // of a SIMD always wins: it runs ahead and the youngest finishes
                // alone, holding up the workgroup's end.  So a wave's issue
                // priority falls from 3 to 0 as it works through a body's tiles,
                // and the SIMD's VALU goes to the waves that are behind
                // (measured on 14336x4096: 12.1 -> 10.8 us at M = 1, 13.5 ->
                // 12.8 us at M = 16; bodies of one tile are left alone: falling
                // over the bodies measured 0.2-0.4 us slower on 4096x14336; so
                // are the 16-wave kernels of 17..32 x rows: 19.2 -> 21.8 us at
                // M = 24).
                if constexpr (TPW > 1 && (MT <= 16 || MT > ST_W16_MAX_M))
                    st_prio(3 - (4 * u) / TPW);
                const bool live = gi * NBG + b < nblk && c < kend;
                const u32x4_t p = pb[u % D];
                const uint32_t sv = slot4 | (live ? static_cast<uint32_t>(b >> 1) << 16 : L.zero);
                u32x4_t bw[4];
                if constexpr (A2) {
                    // bytes 2*s4 and 2*s4+1: four weights each, one 64-bit read
                    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
                    for (int bi = 0; bi < 8; ++bi) {
                        const u32x2_t qv = lds_at<u32x2_t>(
                            smem, __builtin_amdgcn_perm(p[bi >> 2], sv, 0x0C020000u | ((4u + (bi & 3)) << 8)) +
                                      (b & 1) * 128);
                        bw[bi >> 1][2 * (bi & 1)] = qv[0];
                        bw[bi >> 1][2 * (bi & 1) + 1] = qv[1];
                    }
                } else if constexpr (!I4) {
                    // the pair bytes of the four B operands (any3: the fourth from the top bits)
                    const u32x4_t pd = A3 ? u32x4_t{p[0], p[1], p[2], any3_top_pairs(p)} : p;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                        for (int jb = 0; jb < 4; ++jb)
                            bw[s4][jb] = lds_at<uint32_t>(
                                smem, __builtin_amdgcn_perm(pd[s4], sv, 0x0C020000u | ((4u + jb) << 8)) +
                                          (b & 1) * 128);
                }
                const uint32_t pr =
                    lds_at<uint32_t>(smem, L.ab + b * GS * 64 + (min(grp - gbase, GS - 1) * 16 + j) * 4) &
                    (live ? 0xFFFFFFFFu : 0u);
                const float a = __builtin_ldexpf(bf16_to_f32(pr & 0xFFFFu), rsc[b]);
                const float bt = bf16_to_f32(pr >> 16);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const u32x4_t w = I4 ? deq_int4(p[s4], a, bt) : deq_quad(bw[s4], a, bt);
                    const u32x4_t& xa = XL ? xv[s4] : xq[XL ? 0 : s][0][s4];
                    if constexpr (VD) {
                        // v_dot2_f32_bf16: the lane's own two weights times its two x values
                        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t wt = w[t], xt = xa[t];
                            dacc[b] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2_t, wt), __builtin_bit_cast(bf16x2_t, xt),
                                dacc[b], false);
                        }
                    } else {
                        acc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, w),
                            acc[b][0], 0, 0, 0);
#pragma unroll
                        for (int ms = 1; ms < MS; ++ms)
                            acc[b][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, xq[XL ? 0 : s][ms][s4]),
                                __builtin_bit_cast(bf16x8_t, w), acc[b][ms], 0, 0, 0);
                    }
                }
                issue_next(k, u);
            }
        }
        if (k == 0)
            stamp(5);
        __builtin_amdgcn_s_setprio(0);
        if (kb == bpg - 1) {
            // end of a group: partial sums through LDS, y, then the next group's
            // tables.  Only the outputs of rows m < M are passed on: lane l holds
            // y[4*(l/16) + v][l % 16], so the first 16*LQ lanes and VC values.
            stamp(6);
            constexpr int VC = MTS < 4 ? MTS : 4;
            constexpr int LQ = (MTS + 3) / 4;
            constexpr int OUT = 16 * LQ * VC;   // outputs of a block's slice
            float* redf = reinterpret_cast<float*>(smem);
            if constexpr (VD) {
                // the four lanes of a row (l, l+16, l+32, l+48) hold its four
                // k quarters: add them, as the matrix core's output would be
#pragma unroll
                for (int b = 0; b < NBG; ++b) {
                    float t = dacc[b] + __shfl_xor(dacc[b], 16);
                    t += __shfl_xor(t, 32);
                    acc[b][0] = f32x4_t{t, 0.f, 0.f, 0.f};
                    dacc[b] = 0.f;
                }
            }
            // one pass per slice of 16 x rows (the partial sums of one slice
            // fill the table region)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                __syncthreads();
                if (lane < 16 * LQ) {
#pragma unroll
                    for (int b = 0; b < NBG; ++b)
#pragma unroll
                        for (int v = 0; v < VC; ++v)
                            redf[(b * NW + wave) * OUT + lane * VC + v] = acc[b][ms][v];
                }
                if constexpr (MG) {
                    if (ms == 0 && gi + 1 < ngroups)
                        stage_store(lqn, aqn, bqn);
                }
                __syncthreads();
                for (int t = tid; t < NBG * OUT; t += NT) {   // every thread sums outputs
                    const int b = t / OUT;
                    const int o = t - b * OUT;
                    const int blk = gi * NBG + b;
                    float tot = redf[b * NW * OUT + o];
                    for (int w = 1; w < NW; ++w)
                        tot += redf[(b * NW + w) * OUT + o];
                    const int l = o / VC;
                    const int m = 16 * ms + (l >> 4) * 4 + (o - l * VC);
                    const int n = (r + blk * Gs) * TILE_ROWS + (l & 15);
                    if (blk < nblk && m < M && n < N) {
                        if (S > 1)   // this split's partial sum, added up by k_split_sum
                            args.ws[(static_cast<size_t>(split) * M + m) * N + n] = tot;
                        else
                            args.y[static_cast<size_t>(m) * N + n] =
                                static_cast<uint16_t>(f32_to_bf16(tot));
                    }
                }
            }
            stamp(7);
            if constexpr (MG) {
                if (gi + 1 < ngroups) {
                    __syncthreads();
                    build();
                    __syncthreads();
                    load_scales();
#pragma unroll
                    for (int b = 0; b < NBG; ++b)
#pragma unroll
                        for (int ms = 0; ms < MS; ++ms)
                            acc[b][ms] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
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

constexpr int KM_GRID = 256;   // one workgroup per CU of an MI355X

template <int MT, int FMT>
bool launch_st(const GemmArgs& a, hipStream_t stream, unsigned long long* ts);
#ifdef ANY4_PROBE_TS
bool st_disable = false;   // probe builds: time the older kernels
#endif

// k_gemm_st where it measured faster than k_gemm_km / k_gemm_kb: up to four
// row blocks per workgroup (one group).  (One block with K <= 4096 went to
// k_gemm_km until the streaming kernel's early table build: now 6.3 -> 6.0 us
// on 4096x4096 at M = 1, 7.9 -> 6.3 us on 4096x2048 at M = 16.)
bool use_st(const GemmArgs& a)
{
    const int64_t NB = row_blocks(a.N);
    const int64_t grid = NB < KM_GRID ? NB : KM_GRID;
    const int64_t nb = grid > 0 ? (NB + grid - 1) / grid : 0;
    return nb >= 1 && nb <= 4;
}

template <int MT, int FMT>
void launch_gemm(const GemmArgs& a, hipStream_t stream)
{
#ifdef ANY4_PROBE_TS
    if (!st_disable)
#endif
    if (use_st(a) && launch_st<MT, FMT>(a, stream, nullptr))
        return;
    const int64_t NB = row_blocks(a.N);
    int64_t grid = NB < KM_GRID ? NB : KM_GRID;
    if (grid * KM_MAX_BLK < NB)
        grid = (NB + KM_MAX_BLK - 1) / KM_MAX_BLK;
    const int64_t nb = (NB + grid - 1) / grid;                // row blocks per workgroup
    int64_t groups = (nb + 3) / 4;
    int64_t nbg = (nb + groups - 1) / groups;                 // ... decoded together
    const dim3 gd(static_cast<unsigned>(grid));
    if (a.K <= KM_MAX_K) {
        if (nbg == 1)
            hipLaunchKernelGGL((k_gemm_km<MT, 1, FMT>), gd, dim3(GT), 0, stream, a);
        else if (nbg == 2)
            hipLaunchKernelGGL((k_gemm_km<MT, 2, FMT>), gd, dim3(GT), 0, stream, a);
        else if (nbg == 3)
            hipLaunchKernelGGL((k_gemm_km<MT, 3, FMT>), gd, dim3(GT), 0, stream, a);
        else
            hipLaunchKernelGGL((k_gemm_km<MT, 4, FMT>), gd, dim3(GT), 0, stream, a);
        return;
    }
    // alpha/beta of a group must fit the LDS staging of k_gemm_kb
    const int64_t G = a.K / a.g;
    while (nbg > 1 && G > (nbg == 4 ? KbCfg<4, false>::GMAX
                                    : nbg == 3 ? KbCfg<3, false>::GMAX : KbCfg<2, false>::GMAX))
        --nbg;
    // x in LDS: M <= 2, one block per group, and x small enough (measured:
    // with two blocks per group the staging costs more than it saves, e.g.
    // 16.2 against 14.6 us on 8192x8192 at M = 1)
    const bool xl = MT <= 2 && nbg == 1 &&
                    static_cast<int64_t>(a.M) * a.K * 2 <= KbCfg<1, true>::XMAX;
    if (xl) {
        if constexpr (MT <= 2)
            hipLaunchKernelGGL((k_gemm_kb<MT, 1, true, FMT>), gd, dim3(GT), 0, stream, a);
        return;
    }
    if (nbg == 1)
        hipLaunchKernelGGL((k_gemm_kb<MT, 1, false, FMT>), gd, dim3(GT), 0, stream, a);
    else if (nbg == 2)
        hipLaunchKernelGGL((k_gemm_kb<MT, 2, false, FMT>), gd, dim3(GT), 0, stream, a);
    else if (nbg == 3)
        hipLaunchKernelGGL((k_gemm_kb<MT, 3, false, FMT>), gd, dim3(GT), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_kb<MT, 4, false, FMT>), gd, dim3(GT), 0, stream, a);
}

// ---- k_split_sum: y = bf16(sum over splits of the partial sums) ------------
// The partial sums of the S <= 4 workgroups that split K, added in split
// order (so the result does not depend on which workgroup finished first),
// then rounded once to bf16.  ws is [S][M][N] fp32.  Each thread takes four
// consecutive outputs and issues the loads of every split before the first
// add: the partial sums come from other XCDs' writes, so each load is a trip
// past L2, and S dependent trips cost S latencies.  vec: 16-byte loads and
// 8-byte stores (mn a multiple of 4, ws 16-byte and y 8-byte aligned).
constexpr int SPLIT_MAX = 4;

__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ ws,
                                                   uint16_t* __restrict__ y, int S, size_t mn,
                                                   int vec)
{
    const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i >= mn)
        return;
    if (vec) {
        float4 v[SPLIT_MAX] = {};
#pragma unroll
        for (int s = 0; s < SPLIT_MAX; ++s)
            if (s < S)
                v[s] = *reinterpret_cast<const float4*>(ws + static_cast<size_t>(s) * mn + i);
        float4 t = v[0];
#pragma unroll
        for (int s = 1; s < SPLIT_MAX; ++s)
            if (s < S) {
                t.x += v[s].x;
                t.y += v[s].y;
                t.z += v[s].z;
                t.w += v[s].w;
            }
        uint2 o;
        o.x = f32_to_bf16(t.x) | (f32_to_bf16(t.y) << 16);
        o.y = f32_to_bf16(t.z) | (f32_to_bf16(t.w) << 16);
        *reinterpret_cast<uint2*>(y + i) = o;
        return;
    }
    const int n = mn - i < 4 ? static_cast<int>(mn - i) : 4;
    float v[SPLIT_MAX][4] = {};
#pragma unroll
    for (int s = 0; s < SPLIT_MAX; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s < S && j < n)
                v[s][j] = ws[static_cast<size_t>(s) * mn + i + j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float t = v[0][j];
#pragma unroll
        for (int s = 1; s < SPLIT_MAX; ++s)
            if (s < S)
                t += v[s][j];
        if (j < n)
            y[i + j] = static_cast<uint16_t>(f32_to_bf16(t));
    }
}

// ---- k_gemm_st launch: the shape decides waves, blocks per group and ring --
struct StPlan {
    int grid, nw, nbg, r, cw, splits, gstage;
    bool mg, xl;
    StLayout L;
};

// Split K over S workgroups when x, read once per workgroup for all of the
// workgroup's K, would cost more than the weights: the x rows the kernel
// loads (M rounded up to the instantiated 1, 2, 4, 8 or 16; the loads are
// full-width whatever M) times K times 2 bytes against the nb * 16 rows x K
// half-bytes of its row blocks, i.e. more than 4 * nb x rows, with one or two
// row blocks per CU and K of 12288 or more; then each workgroup takes four
// row blocks over K/S.  Needs a workspace of S*M*N fp32 partial sums.
// (Measured at M = 16: 4096x14336 20.4 -> 16.8 us, 8192x28672 45.7 -> 37.4
// us; 8192x8192 gained nothing.  At the threshold, split against unsplit:
// 4096x14336 M = 4 12.9 / 12.4 us, M = 8 13.1 / 15.1; 8192x28672 M = 4
// 33.6 / 29.2, M = 8 32.9 / 31.9, M = 16 35.4 / 44.7.)
inline int st_splits(int M, int N, int K)
{
    const int NB = static_cast<int>(row_blocks(N));
    const int grid = NB < KM_GRID ? NB : KM_GRID;
    const int nb = grid > 0 ? (NB + grid - 1) / grid : 0;
    const int mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    if (mt <= 4 * nb || nb < 1 || nb > 2 || K / TILE_K < 96 || NB < KM_GRID)
        return 1;
    return 4 / nb;
}

size_t st_workspace_bytes(int M, int N, int K)
{
    const int S = st_splits(M, N, K);
    return S > 1 ? static_cast<size_t>(S) * M * N * sizeof(float) : 0;
}

// Ring depths that fit 128 VGPRs (16 waves per CU) without spilling: x in
// the ring costs 16 registers per chunk, the next group's staging 20.  Wide
// batches (ms slices of 16 x rows, 8 waves per CU and 256 VGPRs) take 16*ms
// registers of x per chunk and 4*ms of sums per block.
// The most waves per workgroup: 16 (128 VGPRs each) up to 32 x rows, 8 (256
// VGPRs) beyond, and for two or three slices of x with one block per group
// (its two-step bodies do not fit 128)
constexpr int st_waves(int M, int nbg)
{
    return M > ST_W16_MAX_M || (M > 16 && nbg == 1) ? ST_MAX_WAVES / 2 : ST_MAX_WAVES;
}
constexpr bool st_ring_ok(int nbg, int r, bool xl, bool mg, int ms = 1)
{
    const int tpw = nbg * r;
    if (ms > 1)
        return !xl && !mg && tpw <= 8 && r <= 2;
    if (xl)
        return tpw <= (mg ? 4 : 8);
    if (mg)
        return r == 1 && tpw <= 2;
    return nbg == 1 ? r <= 4 : tpw <= 8 && r <= 2;
}

// Blocks per group, waves, body length and chunks per wave: the fewest dead
// chunks, then the most waves, then the fewest bodies; x in LDS for M <= 2
// where it fits.
#ifdef ANY4_PROBE_TS
int st_force_nw = 0, st_force_r = 0;
#endif
inline bool st_plan(int M, int N, int K, int g, bool split_ok, StPlan& P)
{
    const int NB = static_cast<int>(row_blocks(N));
    const int G = K / g;
    P.splits = split_ok ? st_splits(M, N, K) : 1;
    const int Kc = (K / TILE_K + P.splits - 1) / P.splits;   // chunks of one split
    const int gcn = g / TILE_K;
    // alpha/beta groups a split's chunks touch (its first chunk need not start a group)
    const int gtouch = (Kc + gcn - 1) / gcn + 1;
    P.gstage = P.splits > 1 && gtouch < G ? gtouch : G;
    const int gs = NB * P.splits < KM_GRID ? NB : KM_GRID / P.splits;   // workgroups per split
    P.grid = gs * P.splits;
    const int nb = (NB + gs - 1) / gs;
    for (int nbg = nb <= 1 ? 1 : nb <= 2 ? 2 : 4; nbg >= 1; nbg /= 2) {
        const bool mg = nb > nbg;
        for (int xi = M <= 2 ? 0 : 1; xi < 2; ++xi) {
            const bool xl = xi == 0;
            const StLayout L = st_layout(nbg, P.gstage, M, K, xl);
            if (L.total > ST_LDS)
                continue;
            int best = -1;
            const int ms = M > 16 ? (M + 15) / 16 : 1;
            const int max_waves = st_waves(M, nbg);
            for (int r = 1; r * nbg <= 8; r *= 2) {
                if (!st_ring_ok(nbg, r, xl, mg, ms))
                    continue;
                for (int nw = max_waves; nw >= 1; --nw) {
#ifdef ANY4_PROBE_TS
                    if ((st_force_nw && nw != st_force_nw) || (st_force_r && r != st_force_r))
                        continue;
#endif
                    const int nt = 64 * nw;
                    if (nbg * 2 * G > 2 * nt)
                        continue;
                    if (xl && static_cast<int64_t>(M) * K * 2 > static_cast<int64_t>(ST_XP) * nt * 16)
                        continue;
                    const int cw = r * ((Kc + nw * r - 1) / (nw * r));
                    const int waste = nw * cw - Kc;
                    // x in LDS, one block per group: bodies of a single tile
                    // (a ring of one tile, no falling priority) measured slow,
                    // 11.4 against 9.8 us on 4096x14336 at M = 1 for 16 waves x
                    // 7 one-tile bodies against 14 waves x one 8-tile body
                    const int one_tile = xl && nbg * r == 1 && cw > 1 ? 2048 : 0;
                    const int score = waste * 4096 + one_tile + (max_waves - nw) * 64 + cw / r;
                    if (best < 0 || score < best) {
                        best = score;
                        P.nw = nw;
                        P.r = r;
                        P.cw = cw;
                    }
                }
            }
            if (best >= 0) {
                P.nbg = nbg;
                P.mg = mg;
                P.xl = xl;
                P.L = L;
                return true;
            }
        }
    }
    return false;
}

// Ring tiles issued before the staging data is waited for, and ring depth
// (tiles in flight per wave).  Measured on the 14336x4096 and 4096x14336
// layers: a wave that issues more loads than the CU accepts stalls at issue
// (8 at once: ~6K cycles), while 2 per wave of 16 (32 KB per CU) never
// stall and already keep HBM near its streaming rate; tiles requested ahead
// of the staging loads delay the table build more than they save.
#ifndef ANY4_ST_PRE
#define ANY4_ST_PRE 0
#endif
#ifndef ANY4_ST_D
#define ANY4_ST_D 2
#endif
// The deepest ring up to dw tiles that divides a body and, with x in the
// ring, does not overwrite a step's x before the step's last tile.
constexpr int st_depth(int tb, int nbg, bool xl, int dw)
{
    for (int d = dw < tb ? dw : tb; d > 1; --d)
        if (tb % d == 0 && (xl || tb - d >= nbg - 1))
            return d;
    return 1;
}

template <int MT, int NBG, int R, bool XL, bool MG, int FMT>
void st_go(const StArgs& sa, const StPlan& P, hipStream_t stream)
{
    // 8 waves of 256 VGPRs, 4 tiles in flight each: see st_waves
    constexpr bool W8 = st_waves(MT, NBG) < ST_MAX_WAVES;
    constexpr int LB = W8 ? 512 : 1024;
    constexpr int D = st_depth(NBG * R, NBG, XL, W8 ? 4 : ANY4_ST_D);
    hipLaunchKernelGGL((k_gemm_st<MT, NBG, R, XL, MG, LB, ANY4_ST_PRE, D, FMT>), dim3(P.grid),
                       dim3(64 * P.nw), 0, stream, sa);
}

template <int MT, int NBG, int R, int FMT>
void st_go_r(const StArgs& sa, const StPlan& P, hipStream_t stream)
{
    if constexpr (MT <= 2) {
        if (P.xl) {
            if (P.mg)
                st_go<MT, NBG, R, true, true, FMT>(sa, P, stream);
            else
                st_go<MT, NBG, R, true, false, FMT>(sa, P, stream);
            return;
        }
    }
    if (P.mg)
        st_go<MT, NBG, R, false, true, FMT>(sa, P, stream);
    else
        st_go<MT, NBG, R, false, false, FMT>(sa, P, stream);
}

// The kernel arguments of a plan, with the launch constants worked out here
StArgs st_args(const GemmArgs& a, const StPlan& P, unsigned long long* ts)
{
    StArgs sa;
    sa.a = a;
    sa.splits = P.splits;
    sa.gstage = P.gstage;
    sa.cw = P.cw;
    sa.L = P.L;
    sa.ts = ts;
    const int NB = static_cast<int>(row_blocks(a.N));
    const int Kc = a.K / TILE_K;
    sa.G = a.K / a.g;
    sa.gc = a.g / TILE_K;
    sa.Gs = P.grid / P.splits;
    sa.KcS = (Kc + P.splits - 1) / P.splits;
    sa.nbmax = (NB + sa.Gs - 1) / sa.Gs;
    for (int i = 0; i < 4; ++i)
        sa.gbase[i] = i < P.splits ? i * sa.KcS / sa.gc : 0;
    sa.inv_abper = 1.0f / static_cast<float>(2 * sa.G);
    sa.inv_G = 1.0f / static_cast<float>(sa.G);
    return sa;
}

// The M = 1 product with v_dot2_f32_bf16 instead of the matrix cores (same
// decode, ring and staging); kept to compare the two.
bool launch_st_dot(const GemmArgs& a, hipStream_t stream)
{
    StPlan P;
    if (a.M != 1 || !st_plan(1, a.N, a.K, a.g, false, P) || !P.xl || P.mg)
        return false;
    const StArgs sa = st_args(a, P, nullptr);
    const dim3 gd(P.grid), bd(64 * P.nw);
#define ST_DOT(NBG_, R_)                                                                          \
    hipLaunchKernelGGL((k_gemm_st<1, NBG_, R_, true, false, 1024, ANY4_ST_PRE,                    \
                                  (ANY4_ST_D < NBG_ * R_ ? ANY4_ST_D : NBG_ * R_), FMT_ANY4, true>), \
                       gd, bd, 0, stream, sa)
    switch (P.nbg * 16 + P.r) {
    case 16 + 1: ST_DOT(1, 1); break;
    case 16 + 2: ST_DOT(1, 2); break;
    case 16 + 4: ST_DOT(1, 4); break;
    case 16 + 8: ST_DOT(1, 8); break;
    case 32 + 1: ST_DOT(2, 1); break;
    case 32 + 2: ST_DOT(2, 2); break;
    case 32 + 4: ST_DOT(2, 4); break;
    case 64 + 1: ST_DOT(4, 1); break;
    case 64 + 2: ST_DOT(4, 2); break;
    default: return false;
    }
#undef ST_DOT
    return true;
}

template <int MT, int FMT>
bool launch_st(const GemmArgs& a, hipStream_t stream, unsigned long long* ts)
{
    StPlan P;
    if (!st_plan(a.M, a.N, a.K, a.g, a.ws != nullptr, P))
        return false;
    const StArgs sa = st_args(a, P, ts);
    if constexpr (MT > 16) {
        // wide batches: one group, x in the ring, bodies of one or two steps
        if (P.mg || P.xl || P.splits > 1)
            return false;
        switch (P.nbg * 16 + P.r) {
        case 16 + 1: st_go<MT, 1, 1, false, false, FMT>(sa, P, stream); break;
        case 16 + 2: st_go<MT, 1, 2, false, false, FMT>(sa, P, stream); break;
        case 32 + 1: st_go<MT, 2, 1, false, false, FMT>(sa, P, stream); break;
        case 32 + 2: st_go<MT, 2, 2, false, false, FMT>(sa, P, stream); break;
        case 64 + 1: st_go<MT, 4, 1, false, false, FMT>(sa, P, stream); break;
        case 64 + 2: st_go<MT, 4, 2, false, false, FMT>(sa, P, stream); break;
        default: return false;
        }
        return true;
    } else {
        switch (P.nbg * 16 + P.r) {
        case 16 + 1: st_go_r<MT, 1, 1, FMT>(sa, P, stream); break;
        case 16 + 2: st_go_r<MT, 1, 2, FMT>(sa, P, stream); break;
        case 16 + 4: st_go_r<MT, 1, 4, FMT>(sa, P, stream); break;
        case 16 + 8: st_go_r<MT, 1, 8, FMT>(sa, P, stream); break;
        case 32 + 1: st_go_r<MT, 2, 1, FMT>(sa, P, stream); break;
        case 32 + 2: st_go_r<MT, 2, 2, FMT>(sa, P, stream); break;
        case 32 + 4: st_go_r<MT, 2, 4, FMT>(sa, P, stream); break;
        case 64 + 1: st_go_r<MT, 4, 1, FMT>(sa, P, stream); break;
        case 64 + 2: st_go_r<MT, 4, 2, FMT>(sa, P, stream); break;
        default: return false;
        }
    }
    if (P.splits > 1) {
        const size_t mn = static_cast<size_t>(a.M) * a.N;
        const int vec = mn % 4 == 0 && (reinterpret_cast<uintptr_t>(a.ws) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(a.y) & 7) == 0;
        hipLaunchKernelGGL(k_split_sum, dim3(static_cast<unsigned>((mn + 1023) / 1024)), dim3(256),
                           0, stream, a.ws, a.y, P.splits, mn, vec);
    }
    return true;
}

}  // namespace

// M = 1..16: the streaming kernels, instantiated for 1, 2, 4, 8 and 16 rows
template <int FMT>
static void launch_decode_fmt(const GemmArgs& a, hipStream_t stream)
{
    if (a.M == 1)
        launch_gemm<1, FMT>(a, stream);
    else if (a.M == 2)
        launch_gemm<2, FMT>(a, stream);
    else if (a.M <= 4)
        launch_gemm<4, FMT>(a, stream);
    else if (a.M <= 8)
        launch_gemm<8, FMT>(a, stream);
    else
        launch_gemm<16, FMT>(a, stream);
}

// M = 17..48 in one pass of the streaming kernel (32 or 48 rows), where it
// runs for the shape; false: the caller takes 16-row slices instead
template <int FMT>
static bool launch_wide_fmt(const GemmArgs& a, hipStream_t stream)
{
    if (!use_st(a))
        return false;
    return a.M <= 32 ? launch_st<32, FMT>(a, stream, nullptr) : launch_st<48, FMT>(a, stream, nullptr);
}

static bool launch_wide(const GemmArgs& a, int fmt, hipStream_t stream)
{
    if (fmt == FMT_INT4)
        return launch_wide_fmt<FMT_INT4>(a, stream);
    if (fmt == FMT_ANY2)
        return launch_wide_fmt<FMT_ANY2>(a, stream);
    if (fmt == FMT_ANY3)
        return launch_wide_fmt<FMT_ANY3>(a, stream);
    return launch_wide_fmt<FMT_ANY4>(a, stream);
}

static void launch_decode(const GemmArgs& a, int fmt, hipStream_t stream)
{
    if (fmt == FMT_INT4)
        launch_decode_fmt<FMT_INT4>(a, stream);
    else if (fmt == FMT_ANY2)
        launch_decode_fmt<FMT_ANY2>(a, stream);
    else if (fmt == FMT_ANY3)
        launch_decode_fmt<FMT_ANY3>(a, stream);
    else
        launch_decode_fmt<FMT_ANY4>(a, stream);
}

// 64 weight rows per workgroup: 128 (waves of 64 x 64 outputs) measured
// slower, 370 against 294 us at M = 1024 on 14336x4096
template <int BM>
static void launch_big(const GemmArgs& a, int fmt, hipStream_t stream)
{
    constexpr int BN = BIG_BN;
    const dim3 gd(static_cast<unsigned>((a.N + BN - 1) / BN),
                  static_cast<unsigned>((a.M + BM - 1) / BM));
    if (fmt == FMT_ANY2)
        hipLaunchKernelGGL((k_gemm_big<BM, FMT_ANY2, BN>), gd, dim3(256), 0, stream, a);
    else if (fmt == FMT_ANY3)
        hipLaunchKernelGGL((k_gemm_big<BM, FMT_ANY3, BN>), gd, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_big<BM, FMT_ANY4, BN>), gd, dim3(256), 0, stream, a);
}

// ---- prefill: the layer dequantised once, then a plain bf16 GEMM ----------
// From PREFILL_MIN_M x rows on, with a workspace of N*K bf16, the weights are
// dequantised into it by the format's dequant kernel (the exact values
// any4_dequant writes) and y = x * W^T is one bf16 GEMM with fp32
// accumulation from hipBLASLt: a dequant-GEMM kernel would redo the decode
// for every tile of x rows, and at these M the GEMM is bound by the matrix
// cores, where the library's tuned kernels are the faster choice.  Without a
// workspace (or should the library decline the shape) the tiled kernel runs.
#ifndef ANY4_PREFILL_MIN_M
#define ANY4_PREFILL_MIN_M 128
#endif
constexpr int64_t PREFILL_MIN_M = ANY4_PREFILL_MIN_M;

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    return M >= PREFILL_MIN_M ? static_cast<size_t>(N) * static_cast<size_t>(K) * 2 : 0;
}

void launch_dequant_fmt(int fmt, const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                        const uint16_t* beta, uint16_t* w, int N, int K, int g, hipStream_t stream)
{
    const int64_t Kc = K / TILE_K;
    const dim3 gd(static_cast<unsigned>(row_blocks(N) * ((Kc + DQ_WAVES - 1) / DQ_WAVES)));
    if (fmt == FMT_ANY2)
        hipLaunchKernelGGL(k_dequant2, gd, dim3(64 * DQ_WAVES), 0, stream, packed, lut, alpha, beta, w,
                           N, K, g);
    else if (fmt == FMT_ANY3)
        hipLaunchKernelGGL(k_dequant3, gd, dim3(64 * DQ_WAVES), 0, stream, packed, lut, alpha, beta, w,
                           N, K, g);
    else
        hipLaunchKernelGGL(k_dequant, gd, dim3(64 * DQ_WAVES), 0, stream, packed, lut, alpha, beta, w,
                           N, K, g, fmt == FMT_INT4 ? 1 : 0);
}

// One hipBLASLt handle per device and one matmul plan per (device, M, N, K),
// made on first use and kept until the process ends (the heuristic query
// is host work worth doing once; making them on first use keeps them out of
// any graph the caller captures later).  On that first use, unless the
// stream is being captured, the library's candidate algorithms (up to
// BLAS_CANDIDATES) are timed on the call's own operands and the fastest is
// kept (measured on 14336x4096, dequant and GEMM: M = 256 64 us against 71
// with the heuristic's first choice; M = 128, 512 and 1024 the same within
// 2%).  ANY4_BLAS_TUNE=0 keeps the first choice.
constexpr int BLAS_CANDIDATES = 16;

struct BlasPlan {
    int dev;
    int64_t M, N, K;
    bool ok;
    hipblasLtMatmulDesc_t desc;
    hipblasLtMatrixLayout_t la, lb, lc;
    hipblasLtMatmulAlgo_t algo;
};
std::mutex blas_mu;
hipblasLtHandle_t blas_handles[64];
std::deque<BlasPlan> blas_plans;   // a deque: a plan stays put while others are added

bool blas_run(const BlasPlan& p, const hipblasLtMatmulAlgo_t& algo, const uint16_t* w,
              const uint16_t* x, uint16_t* y, hipStream_t stream)
{
    const float one = 1.0f, zero = 0.0f;
    return hipblasLtMatmul(blas_handles[p.dev], p.desc, &one, w, p.la, x, p.lb, &zero, y, p.lc, y,
                           p.lc, &algo, nullptr, 0, stream) == HIPBLAS_STATUS_SUCCESS;
}

bool blas_tuning()
{
    const char* e = std::getenv("ANY4_BLAS_TUNE");
    return !(e && e[0] == '0');
}

// The fastest of the n candidates on these operands (five timed runs each,
// after one untimed), kept only when it beats the heuristic's first choice by
// more than 5% (closer than that, the pick follows timing noise); -1 when
// timing is not possible.  y is overwritten.
int blas_pick(const BlasPlan& p, const hipblasLtMatmulHeuristicResult_t* res, int n,
              const uint16_t* w, const uint16_t* x, uint16_t* y, hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return -1;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0)
            (void)hipEventDestroy(e0);
        return -1;
    }
    int best = -1;
    float best_ms = 0.0f, first_ms = 0.0f;
    for (int i = 0; i < n; ++i) {
        if (!blas_run(p, res[i].algo, w, x, y, stream))
            continue;
        bool ok = hipEventRecord(e0, stream) == hipSuccess;
        for (int r = 0; r < 5 && ok; ++r)
            ok = blas_run(p, res[i].algo, w, x, y, stream);
        float ms = 0.0f;
        ok = ok && hipEventRecord(e1, stream) == hipSuccess &&
             hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        if (!ok)
            continue;
        if (i == 0)
            first_ms = ms;
        if (best < 0 || ms < best_ms) {
            best = i;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return first_ms > 0.0f && best_ms > 0.95f * first_ms ? 0 : best;
}

const BlasPlan* blas_plan(int dev, int64_t M, int64_t N, int64_t K, const uint16_t* w,
                          const uint16_t* x, uint16_t* y, hipStream_t stream)
{
    std::lock_guard<std::mutex> lock(blas_mu);
    for (const BlasPlan& p : blas_plans)
        if (p.dev == dev && p.M == M && p.N == N && p.K == K)
            return p.ok ? &p : nullptr;
    BlasPlan p{dev, M, N, K, false, nullptr, nullptr, nullptr, nullptr, {}};
    bool ok = dev >= 0 && dev < 64;
    if (ok && !blas_handles[dev])
        ok = hipblasLtCreate(&blas_handles[dev]) == HIPBLAS_STATUS_SUCCESS;
    // column-major view: Y (N x M, ld N) = op(A) (N x K) * B (K x M), with
    // A = W seen as K x N (ld K) transposed and B = x seen as K x M (ld K)
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    ok = ok && hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS;
    if (ok) {
        // no library workspace: the algorithms that need one are left out
        hipblasLtMatmulPreference_t pref = nullptr;
        uint64_t wsz = 0;
        hipblasLtMatmulHeuristicResult_t res[BLAS_CANDIDATES];
        int n = 0;
        ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
             hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz,
                                                   sizeof(wsz)) == HIPBLAS_STATUS_SUCCESS &&
             hipblasLtMatmulAlgoGetHeuristic(blas_handles[dev], p.desc, p.la, p.lb, p.lc, p.lc, pref,
                                             blas_tuning() ? BLAS_CANDIDATES : 1, res,
                                             &n) == HIPBLAS_STATUS_SUCCESS &&
             n > 0;
        if (ok) {
            const int pick = n > 1 ? blas_pick(p, res, n, w, x, y, stream) : -1;
            p.algo = res[pick >= 0 ? pick : 0].algo;
        }
        if (pref)
            hipblasLtMatmulPreferenceDestroy(pref);
    }
    p.ok = ok;
    blas_plans.push_back(p);
    return ok ? &blas_plans.back() : nullptr;
}

// y = x * W^T through the library; false: not run (the caller falls back)
bool blas_gemm(const uint16_t* w, const uint16_t* x, uint16_t* y, int64_t M, int64_t N, int64_t K,
               hipStream_t stream)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return false;
    const BlasPlan* p = blas_plan(dev, M, N, K, w, x, y, stream);
    return p && blas_run(*p, p->algo, w, x, y, stream);
}

// Argument checks and dispatch shared by any4_gemm (table lookup),
// any4_gemm_int4 (the 4-bit code itself is the value; lut unused), any2_gemm
// and any3_gemm.
static any4_status gemm_call(int fmt, const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, hipStream_t stream,
                      void* workspace = nullptr, size_t workspace_bytes = 0)
{
    const bool i4 = fmt == FMT_INT4;
    if (M < 0 || N < 0 || !group_ok(K, g) || K / (g > 0 ? g : 1) > MAX_G ||
        (M > 16 && (M + 63) / 64 > 65535))
        return ANY4_E_SHAPE;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(M) * K * 2 >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(N) * 32 >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (M == 0 || N == 0)
        return ANY4_OK;
    if (!y || (K > 0 && (!x || !packed || (!i4 && !lut) || !alpha || !beta)))
        return ANY4_E_NULL;
    if (!aligned(y, 2) || (K > 0 && (!aligned(x, 16) || !aligned(packed, 16) ||
                                     (!i4 && !aligned(lut, 16)) || !aligned(alpha, 16) ||
                                     !aligned(beta, 16))))
        return ANY4_E_ALIGN;
    // the workspace is optional: with one, K may be split over workgroups
    // (M <= 16), or the layer is dequantised into it (prefill)
    const size_t need = K == 0 ? 0
                        : M <= 16 ? st_workspace_bytes(static_cast<int>(M), static_cast<int>(N),
                                                       static_cast<int>(K))
                                  : prefill_workspace_bytes(M, N, K);
    if (workspace && workspace_bytes < need)
        return ANY4_E_WORKSPACE;
    if (workspace && !aligned(workspace, 16))
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
    a.ws = need > 0 && workspace && M <= 16 ? static_cast<float*>(workspace) : nullptr;
    a.ws_bytes = a.ws ? workspace_bytes : 0;
    if (need > 0 && workspace && M >= PREFILL_MIN_M) {
        uint16_t* w = static_cast<uint16_t*>(workspace);
        launch_dequant_fmt(fmt, packed, lut, alpha, beta, w, a.N, a.K, a.g, stream);
        if (launched() != ANY4_OK)
            return ANY4_E_HIP;
        if (blas_gemm(w, x, y, M, N, K, stream))
            return launched();
    }
    if (M > 16 && M <= 48) {
        // a few decode batches: one pass of the streaming kernel with two or
        // three 16-row slices of x against each decoded weight tile; for the
        // shapes it does not run, 16-row slices of x and y through the decode
        // kernels (each slice re-reads the weights, still cheaper than the
        // tiled kernel while it cannot fill the chip)
        GemmArgs w = a;
        w.ws = nullptr;   // no split of K
        if (launch_wide(w, fmt, stream))
            return launched();
        for (int64_t m0 = 0; m0 < M; m0 += 16) {
            GemmArgs s16 = a;
            s16.x = x + m0 * K;
            s16.y = y + m0 * N;
            s16.ws = nullptr;   // the slices do not split K
            s16.M = static_cast<int>(M - m0 < 16 ? M - m0 : 16);
            launch_decode(s16, fmt, stream);
        }
        return launched();
    }
    if (M > 16) {
        // the tiled kernel; int4 is its 4-bit path with no table (lut null)
        if (M <= 64)
            launch_big<64>(a, fmt, stream);
        else
            launch_big<128>(a, fmt, stream);
        return launched();
    }
    launch_decode(a, fmt, stream);
    return launched();
}

// any2 / any3 pack and dequant: checks as any4_pack / any4_dequant, then
// the kernel of the format (bits = 2 or 3).
static any4_status lowbit_pack(int bits, const uint8_t* idx, uint8_t* packed, int64_t N,
                               int64_t K, hipStream_t stream)
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
    const size_t slot_bytes = bits == 2 ? 8 : 12;
    const size_t nbytes = bits == 2 ? any2_packed_bytes(N, K) : any3_packed_bytes(N, K);
    const uint32_t slots = static_cast<uint32_t>(nbytes / slot_bytes);
    const uint32_t blocks = (slots + PACK_THREADS - 1) / PACK_THREADS;
    (void)hipGetLastError();
    if (bits == 2)
        hipLaunchKernelGGL(k_pack2, dim3(blocks), dim3(PACK_THREADS), 0, stream, idx, packed,
                           static_cast<int>(N), static_cast<int>(K), slots);
    else
        hipLaunchKernelGGL(k_pack3, dim3(blocks), dim3(PACK_THREADS), 0, stream, idx, packed,
                           static_cast<int>(N), static_cast<int>(K), slots);
    return launched();
}

static any4_status lowbit_dequant(int bits, const uint8_t* packed, const uint16_t* lut,
                                  const uint16_t* alpha, const uint16_t* beta, uint16_t* w,
                                  int64_t N, int64_t K, int64_t g, hipStream_t stream)
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
    const dim3 gd(static_cast<unsigned>(row_blocks(N) * ((Kc + DQ_WAVES - 1) / DQ_WAVES)));
    (void)hipGetLastError();
    if (bits == 2)
        hipLaunchKernelGGL(k_dequant2, gd, dim3(64 * DQ_WAVES), 0, stream, packed, lut, alpha,
                           beta, w, static_cast<int>(N), static_cast<int>(K),
                           static_cast<int>(g));
    else
        hipLaunchKernelGGL(k_dequant3, gd, dim3(64 * DQ_WAVES), 0, stream, packed, lut, alpha,
                           beta, w, static_cast<int>(N), static_cast<int>(K),
                           static_cast<int>(g));
    return launched();
}

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// allocation-free GEMM: the split-K partial sums in a static device array
// ---------------------------------------------------------------------------
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel: in
// host code that name is only a stand-in for the device symbol, so its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept in scratch_ptr.
constexpr size_t SCRATCH_BYTES = static_cast<size_t>(4) << 20;   // 4 MiB per GPU
static __device__ __attribute__((aligned(256))) uint8_t scratch[SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[SCRATCH_DEVICES];

// The current device's copy of `scratch` (looked up on its first use there).
any4_status scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES)
        return ANY4_E_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return ANY4_E_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return ANY4_OK;
}
}  // namespace

extern "C" {

const char* any4_status_string(any4_status s)
{
    switch (s) {
    case ANY4_OK: return "ANY4_OK: success";
    case ANY4_E_NULL: return "ANY4_E_NULL: a required pointer is NULL";
    case ANY4_E_SHAPE: return "ANY4_E_SHAPE: unsupported sizes (negative size, K not a multiple "
                              "of 128, g not a positive multiple of 128, K % g != 0, K/g > 512, "
                              "M above 65535*64, or buffers of 2 GiB or more)";
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
                       static_cast<int>(K), static_cast<int>(g), 0);
    return launched();
}

size_t any4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t g)
{
    if (M <= 0 || N <= 0 || K <= 0 || !group_ok(K, g) ||
        N >= (static_cast<int64_t>(1) << 31) || K >= (static_cast<int64_t>(1) << 31))
        return 0;
    if (M > 16)
        return prefill_workspace_bytes(M, N, K);
    return st_workspace_bytes(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
}

any4_status any4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    return gemm_call(FMT_ANY4, x, packed, lut, alpha, beta, y, M, N, K, g, stream, workspace,
                     workspace_bytes);
}

any4_status any4_gemm_noalloc(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                              const uint16_t* alpha, const uint16_t* beta, uint16_t* y,
                              int64_t M, int64_t N, int64_t K, int64_t g, hipStream_t stream)
{
    // the same kernels as any4_gemm with a workspace of
    // any4_gemm_workspace_size bytes, that workspace being this GPU's scratch
    // (M <= 16; larger batches run as any4_gemm without a workspace)
    const size_t need = M <= 16 ? any4_gemm_workspace_size(M, N, K, g) : 0;
    if (need > SCRATCH_BYTES)
        return ANY4_E_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const any4_status st = scratch_of_current_device(&ws);
        if (st != ANY4_OK)
            return st;
    }
    return gemm_call(FMT_ANY4, x, packed, lut, alpha, beta, y, M, N, K, g, stream, ws, need);
}

any4_status any4_gemv_dot(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                          const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t N,
                          int64_t K, int64_t g, hipStream_t stream)
{
    if (N < 0 || !group_ok(K, g) || K == 0 || K / g > MAX_G)
        return ANY4_E_SHAPE;
    if (any4_packed_bytes(N, K) >= (static_cast<size_t>(1) << 31) ||
        static_cast<size_t>(N) * 32 >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (N == 0)
        return ANY4_OK;
    if (!x || !packed || !lut || !alpha || !beta || !y)
        return ANY4_E_NULL;
    if (!aligned(y, 2) || !aligned(x, 16) || !aligned(packed, 16) || !aligned(lut, 16) ||
        !aligned(alpha, 16) || !aligned(beta, 16))
        return ANY4_E_ALIGN;
    GemmArgs a{};
    a.x = x;
    a.packed = packed;
    a.lut = lut;
    a.alpha = alpha;
    a.beta = beta;
    a.y = y;
    a.M = 1;
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.g = static_cast<int>(g);
    (void)hipGetLastError();
    if (!launch_st_dot(a, stream))
        return ANY4_E_SHAPE;   // x does not fit the kernel's LDS staging
    return launched();
}

any4_status any4_gemm_int4(const uint16_t* x, const uint8_t* packed, const uint16_t* alpha,
                           const uint16_t* beta, uint16_t* y, int64_t M, int64_t N, int64_t K,
                           int64_t g, void* workspace, size_t workspace_bytes,
                           hipStream_t stream)
{
    return gemm_call(FMT_INT4, x, packed, nullptr, alpha, beta, y, M, N, K, g, stream, workspace,
                     workspace_bytes);
}

any4_status any4_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream)
{
    if (bytes % 1024 != 0 || bytes >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (bytes == 0)
        return ANY4_OK;
    if (!buf || !out)
        return ANY4_E_NULL;
    if (!aligned(buf, 16) || !aligned(out, 4))
        return ANY4_E_ALIGN;
    const uint32_t tiles = static_cast<uint32_t>(bytes / 1024);
    const uint32_t waves = KM_GRID * PROBE_WAVES;
    uint32_t depth = (tiles + waves - 1) / waves;
    if (depth > PROBE_MAX_DEPTH)
        depth = PROBE_MAX_DEPTH;
    const uint32_t per_wg = PROBE_WAVES * depth;
    uint32_t grid = (tiles + per_wg - 1) / per_wg;
    if (grid > KM_GRID)
        grid = KM_GRID;
    const dim3 gd(grid), bd(64 * PROBE_WAVES);
    const uint8_t* b = static_cast<const uint8_t*>(buf);
    (void)hipGetLastError();
    switch (depth) {
#define PROBE_CASE(D_) \
    case D_: hipLaunchKernelGGL(k_read_probe<D_>, gd, bd, 0, stream, b, tiles, out); break;
    PROBE_CASE(1) PROBE_CASE(2) PROBE_CASE(3) PROBE_CASE(4) PROBE_CASE(5) PROBE_CASE(6)
    PROBE_CASE(7) PROBE_CASE(8) PROBE_CASE(9) PROBE_CASE(10) PROBE_CASE(11) PROBE_CASE(12)
    PROBE_CASE(13) PROBE_CASE(14) PROBE_CASE(15) PROBE_CASE(16)
#undef PROBE_CASE
    default: return ANY4_E_SHAPE;
    }
    return launched();
}

size_t any2_packed_bytes(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % TILE_K != 0)
        return 0;
    return static_cast<size_t>(row_blocks(N)) * TILE_ROWS * static_cast<size_t>(K / 4);
}

size_t any3_packed_bytes(int64_t N, int64_t K)
{
    if (N < 0 || K < 0 || K % TILE_K != 0)
        return 0;
    return static_cast<size_t>(row_blocks(N)) * TILE_ROWS * static_cast<size_t>(K / 8 * 3);
}

any4_status any2_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream)
{
    return lowbit_pack(2, idx, packed, N, K, stream);
}

any4_status any3_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream)
{
    return lowbit_pack(3, idx, packed, N, K, stream);
}

any4_status any2_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream)
{
    return lowbit_dequant(2, packed, lut, alpha, beta, w, N, K, g, stream);
}

any4_status any3_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream)
{
    return lowbit_dequant(3, packed, lut, alpha, beta, w, N, K, g, stream);
}

any4_status any2_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    return gemm_call(FMT_ANY2, x, packed, lut, alpha, beta, y, M, N, K, g, stream, workspace,
                     workspace_bytes);
}

any4_status any3_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    return gemm_call(FMT_ANY3, x, packed, lut, alpha, beta, y, M, N, K, g, stream, workspace,
                     workspace_bytes);
}

any4_status any4_quantize(const float* W, const float* ex, uint8_t* idx, uint16_t* lut,
                          uint16_t* alpha, uint16_t* beta, int64_t N, int64_t K, int64_t g,
                          int iters, int bits, hipStream_t stream)
{
    if (N < 0 || K < 0 || g <= 0 || K % g != 0 || iters < 0 || bits < 2 || bits > 4 ||
        static_cast<size_t>(N) * K >= (static_cast<size_t>(1) << 31))
        return ANY4_E_SHAPE;
    if (N == 0 || K == 0)
        return ANY4_OK;
    if (!W || !ex || !idx || !lut || !alpha || !beta)
        return ANY4_E_NULL;
    if (!aligned(W, 4) || !aligned(ex, 4) || !aligned(lut, 2) || !aligned(alpha, 2) ||
        !aligned(beta, 2))
        return ANY4_E_ALIGN;
    (void)hipGetLastError();
    if (K / g <= QW_MAX_G)
        hipLaunchKernelGGL(k_quantize_w, dim3(static_cast<unsigned>((N + QW_WAVES - 1) / QW_WAVES)),
                           dim3(64 * QW_WAVES), 0, stream, W, ex, idx, lut, alpha, beta,
                           static_cast<int>(N), static_cast<int>(K), static_cast<int>(g), iters,
                           1 << bits);
    else
        hipLaunchKernelGGL(k_quantize, dim3(static_cast<unsigned>((N + QT - 1) / QT)), dim3(QT), 0,
                           stream, W, ex, idx, lut, alpha, beta, static_cast<int>(N),
                           static_cast<int>(K), static_cast<int>(g), iters, 1 << bits);
    return launched();
}

}  // extern "C"
