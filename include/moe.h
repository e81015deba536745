/*
 * moe.h -- C ABI of the MI355X (gfx950) MXFP4 routed-expert MoE layer.
 *
 * One MoE layer of the DeepSeek-V4-Flash shape ("DeepSeek-V4-Flash export
 * design", Source configuration, MoE bullet): hidden H = 4096, E = 256 routed
 * experts, top k = 6, intermediate I = 2048, one shared expert, routing
 * weights normalised and scaled by 1.5, or expert ids from a token-id hash
 * table in the first layers.  The layer is four calls on one HIP stream:
 *
 *   moe_route       x -> (ids [T,k], weights [T,k])
 *   moe_dispatch    ids -> (offsets, row_token, slot_row)
 *   moe_expert_ffn  x, packed MXFP4 experts -> out_rows [rows, H] (bf16)
 *   moe_combine     out_rows, slot_row, weights -> y [T, H] (bf16)
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless a comment says host.  The caller owns
 *    and allocates every buffer, workspaces included; the library never
 *    allocates, frees, prints or aborts.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *    call only enqueues kernels on it and returns; nothing synchronises.
 *  - Arguments are validated on the host before anything is enqueued.  Any
 *    return other than MOE_OK means nothing was enqueued.  MOE_EHIP means a
 *    launch failed (hipGetLastError after the launches); work may have been
 *    enqueued before the failing launch.
 *  - T = 0 is a no-op that returns MOE_OK.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Calls hold no state between them and may run from several host threads;
 *    calls that share an output or workspace buffer on overlapping streams race.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    (no floating-point atomics; every reduction runs in a fixed order).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1u

/* Layout tags of an expert blob.  A blob whose tag is not the one a call
 * expects is refused with MOE_ELAYOUT, so bytes in another layout are never
 * misread (the "fail loudly" convention of "ElytronAI / DeepSeek-v4-Flash",
 * Loading). */
#define MOE_LAYOUT_CANONICAL_MXFP4 0x4D584330u  /* host reference layout, below */
#define MOE_LAYOUT_GFX950_TILED_V1 0x4D584731u  /* device layout read by the kernels */

/*
 * moe_experts.flags.  MOE_FFN_SPLIT_FP8 moves the prefill family of the expert
 * FFN (the token counts that do not take the decode family) onto the gfx950
 * scaled matrix cores, which take the E2M1 weights and their E8M0 scales as
 * stored.  Their other operand must be an 8-bit float, so each bf16
 * activation a (x, then h) is carried as two E4M3 terms under one E8M0 scale
 * S per 32 consecutive k:  a = S * hi + (S / 16) * lo.  That is exact for
 * every value within 2^13 of its block's largest magnitude and off by at
 * most 2^-21 of that magnitude below it (the reading taken for this option
 * of "ElytronAI / DeepSeek-v4-Flash", Sizes, where the experts are MXFP4, and
 * of the activations being bf16: weights stay MXFP4, activations keep bf16
 * precision).  Default 0: the weights are
 * decoded to bf16 for bf16 matrix cores.  The flag changes the workspace size.
 */
#define MOE_FFN_SPLIT_FP8 1

/*
 * moe_experts.flags.  MOE_SHARED_MXFP8: the shared expert (slot n_experts,
 * still at base + n_experts * expert_bytes) is MXFP8 -- one E4M3 code per
 * weight (OCP FP8 without infinities: sign, 4 exponent bits with bias 7, 3
 * mantissa bits; codes 0x7f and 0xff are NaN) times the same E8M0 group-32
 * scales -- and takes moe_expert_bytes_mxfp8(H, I) bytes.  This is the
 * dense-weight format of "ElytronAI / DeepSeek-v4-Flash", Sizes (mxfp8_lt:
 * one E8M0 per 32 columns), read here as the shared expert's precision, an
 * inference the pages leave open.  Not combinable with MOE_FFN_SPLIT_FP8
 * (MOE_EINVAL).
 */
#define MOE_SHARED_MXFP8 2

/*
 * moe_experts.flags.  MOE_ROUTED_AFFINE2: the n_experts routed experts are in
 * the 2-bit affine codec of "OsaurusAI / DeepSeek-V4-Flash-0731-JANG", Dynamic
 * affine recipe: weight = s * q + b with q an unsigned 2-bit code and one bf16
 * scale s and one bf16 bias b per group of 64 consecutive input columns (gate,
 * up) or 32 (down).  expert_bytes must equal moe_expert_bytes_affine2(H, I)
 * (= H * I: 2.5, 2.5 and 3 bits per weight).  The shared expert, slot
 * n_experts at base + n_experts * expert_bytes, keeps an MX layout: MXFP4
 * (moe_expert_bytes(H, I) bytes) or, with MOE_SHARED_MXFP8, MXFP8 -- the
 * recipe's shared expert is 8-bit.  H and I must each be 512, 1024, 2048 or
 * 4096 (MOE_ESHAPE otherwise: the decode kernel family has no other sizes
 * for this codec).  Not combinable with MOE_FFN_SPLIT_FP8 (MOE_EINVAL).
 * The 3-bit gate of six listed layers in the same recipe is not supported.
 */
#define MOE_ROUTED_AFFINE2 4

/* Largest hidden or intermediate size (H, I) any call accepts. */
#define MOE_MAX_DIM 65536

/* Largest token count T any call accepts (MOE_ESHAPE beyond; the workspace
 * size queries return 0): it keeps every launch's grid within the device's
 * limits and every row count T * (top_k + 1) in 32 bits. */
#define MOE_MAX_TOKENS 262144

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,      /* NULL pointer, negative size, inconsistent arguments */
  MOE_EALIGN = 2,      /* a pointer misses its required alignment */
  MOE_ELAYOUT = 3,     /* wrong layout tag or ABI version in a descriptor */
  MOE_ESHAPE = 4,      /* unsupported H, I, E or top_k, or expert_bytes mismatch */
  MOE_EWORKSPACE = 5,  /* workspace smaller than the matching *_workspace_size() */
  MOE_EHIP = 6         /* a HIP launch failed */
} moe_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(int status);

/* Library ABI version (MOE_ABI_VERSION of the build). */
uint32_t moe_abi_version(void);

/*
 * Expert weights: MXFP4 ("ElytronAI / DeepSeek-v4-Flash", Sizes): every
 * weight is an E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) times the E8M0 scale 2^(e-127) of
 * its group of 32 consecutive input columns.  4.25 bits per weight, no
 * padding.  The experts of a layer sit back to back in one blob with no gap,
 * so expert xid starts at base + xid * expert_bytes (same page, Layout); the
 * shared expert is stored as xid = n_experts.
 *
 * Canonical layout of one expert (host side, the input of moe_pack_mxfp4):
 *   gate [I, H] | up [I, H] | down [H, I]; each projection [N, K] is its
 *   nibble plane uint8 [N][K/2] (byte b of a row: column 2b in bits 3:0,
 *   column 2b+1 in bits 7:4) followed by its scale plane uint8 [N][K/32].
 *
 * Device layout MOE_LAYOUT_GFX950_TILED_V1: the same six planes at the same
 * offsets with the bytes of each plane permuted (a pure permutation, so
 * expert_bytes is unchanged):
 *   nibble plane: 1024-byte tiles t = (n/16) * (K/128) + (k/128); inside a
 *     tile, lane l = 16*g + r (r < 16, g < 4) owns bytes [16l, 16l+16): the
 *     canonical bytes of row 16*(n/16) + r covering columns
 *     128*(k/128) + 32*g .. +31, in canonical nibble order.
 *   scale plane: 256-byte blocks b = (n/16) * (K/512) + (k/512); byte 4l+i of
 *     a block is the scale of row 16*(n/16) + (l%16) for the 32-column group
 *     16*(k/512) + 4*i + (l/16).
 * One 64-lane wave reads a tile with one coalesced 16-byte load per lane and
 * holds exactly the 32 codes, and the one scale, that its MFMA fragments need.
 *
 * An MXFP8 expert (MOE_SHARED_MXFP8) has the same three projections, each its
 * code plane uint8 [N][K] (one E4M3 byte per weight, row-major) followed by
 * its scale plane uint8 [N][K/32], canonically; in the device layout the code
 * plane is cut into 2048-byte tiles t = (n/16) * (K/128) + (k/128), and inside
 * a tile lane l = 16*g + r owns bytes [16l, 16l+16) (columns 128*(k/128) +
 * 32*g .. +15 of row 16*(n/16) + r) and bytes [1024 + 16l, 1024 + 16l + 16)
 * (columns +16 .. +31); the scale plane is tiled exactly as above.
 */
/*
 * A 2-bit affine expert (MOE_ROUTED_AFFINE2) has the three projections gate
 * [I, H] (group G = 64), up [I, H] (G = 64), down [H, I] (G = 32), each
 * canonically its code plane uint8 [N][K/4] (byte b of a row: column 4b + j
 * in bits 2j+1:2j) followed by its scale plane bf16 [N][K/G] and its bias
 * plane bf16 [N][K/G] (little-endian).  Device layout, per projection at the
 * same offsets:
 *   code plane: 512-byte tiles t = (n/16) * (K/128) + (k/128); inside a tile,
 *     lane l = 16*g + r owns bytes [8l, 8l+8) as two little-endian words; word
 *     u holds the 16 codes of row 16*(n/16) + r at columns 128*(k/128) +
 *     32*s + 8*g + i for s in {2u, 2u+1}, i < 8, code (s, i) in bits
 *     4*i + 2*(s%2) +1 : +0 (so word & 0x33333333 and (word >> 2) &
 *     0x33333333 are eight E2M1 nibbles each, code q read as the value q/2).
 *   scale and bias planes, together: blocks of 16 * (128/G) * 4 bytes, block
 *     (n/16) * (K/128) + (k/128); entry (n%16) * (128/G) + (k%128)/G of a
 *     block is 4 bytes: the bf16 scale, then the bf16 bias, of row n's group
 *     at column k.
 * So one 8-byte load per lane gives a wave the codes of a 16-column x 128-k
 * tile, each run of 8 codes feeding one 16x16x32 MFMA inside a single group.
 */
typedef struct moe_experts {
  uint32_t abi_version;   /* MOE_ABI_VERSION */
  uint32_t layout;        /* MOE_LAYOUT_GFX950_TILED_V1 for the compute calls */
  int32_t n_experts;      /* routed experts E (blob holds E + 1 experts) */
  int32_t hidden;         /* H */
  int32_t inter;          /* I */
  int32_t flags;          /* 0 or MOE_FFN_SPLIT_FP8, MOE_SHARED_MXFP8, MOE_ROUTED_AFFINE2 (see each) */
  uint64_t expert_bytes;  /* moe_expert_bytes(H, I), or moe_expert_bytes_affine2(H, I) */
  const void* base;       /* device pointer, 256-byte aligned */
} moe_experts;

/* Bytes of one expert (gate + up + down) of shape (H, I): 3*H*I*17/32.
 * Returns 0 for unsupported shapes (H, I must be positive multiples of 512,
 * at most MOE_MAX_DIM). */
uint64_t moe_expert_bytes(int32_t hidden, int32_t inter);

/* Fill a descriptor for a device blob in MOE_LAYOUT_GFX950_TILED_V1.
 * MOE_EINVAL for NULL d/base, MOE_ESHAPE for an unsupported shape or E. */
int moe_experts_init(moe_experts* d, const void* base, int32_t n_experts, int32_t hidden, int32_t inter);

/*
 * Host-side repack canonical -> device layout (and back), for n_total experts
 * (routed + shared) of shape (H, I).  src and dst are HOST pointers to
 * n_total * moe_expert_bytes(H, I) bytes each (dst_bytes/src_bytes must be at
 * least that), and must not overlap.  The repack is a pure byte permutation,
 * so unpack(pack(b)) == b exactly (the round trip that "ElytronAI /
 * DeepSeek-v4-Flash", Verification, reports for its own repacked blobs).
 * Synchronous; touches no GPU.
 */
int moe_pack_mxfp4(const uint8_t* src_canonical, uint64_t src_bytes, int32_t n_total, int32_t hidden,
                   int32_t inter, uint8_t* dst_device_layout, uint64_t dst_bytes);
int moe_unpack_mxfp4(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t n_total, int32_t hidden,
                     int32_t inter, uint8_t* dst_canonical, uint64_t dst_bytes);

/* Bytes of one MXFP8 expert of shape (H, I): 3*H*I*33/32; 0 for unsupported shapes. */
uint64_t moe_expert_bytes_mxfp8(int32_t hidden, int32_t inter);

/*
 * The same repack for ONE MXFP8 expert (the MOE_SHARED_MXFP8 shared expert):
 * src and dst are HOST pointers to moe_expert_bytes_mxfp8(H, I) bytes each,
 * not overlapping; a pure byte permutation, so unpack(pack(b)) == b.  A
 * device blob with an MXFP8 shared expert is the E packed MXFP4 experts
 * followed by this expert's packed bytes.
 */
int moe_pack_mxfp8(const uint8_t* src_canonical, uint64_t src_bytes, int32_t hidden, int32_t inter,
                   uint8_t* dst_device_layout, uint64_t dst_bytes);
int moe_unpack_mxfp8(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t hidden, int32_t inter,
                     uint8_t* dst_canonical, uint64_t dst_bytes);

/* Bytes of one 2-bit affine expert of shape (H, I): H * I; 0 for unsupported shapes. */
uint64_t moe_expert_bytes_affine2(int32_t hidden, int32_t inter);

/*
 * Repack of n_experts 2-bit affine routed experts, canonical <-> device
 * layout: src and dst are HOST pointers to n_experts *
 * moe_expert_bytes_affine2(H, I) bytes each, not overlapping.  A permutation
 * of the 2-bit codes and of the (scale, bias) pairs, so unpack(pack(b)) == b.
 * A device blob with affine routed experts is their packed bytes followed by
 * the packed MX shared expert (moe_pack_mxfp4 with n_total = 1, or
 * moe_pack_mxfp8).  Synchronous; touches no GPU.
 */
int moe_pack_affine2(const uint8_t* src_canonical, uint64_t src_bytes, int32_t n_experts, int32_t hidden,
                     int32_t inter, uint8_t* dst_device_layout, uint64_t dst_bytes);
int moe_unpack_affine2(const uint8_t* src_device_layout, uint64_t src_bytes, int32_t n_experts, int32_t hidden,
                       int32_t inter, uint8_t* dst_canonical, uint64_t dst_bytes);

/*
 * Routing ("Model techniques map -- DeepSeek-V4-Flash", Checked in its code,
 * rows "Mixture of experts" and "Auxiliary-loss-free load balancing";
 * "DeepSeek-V4-Flash export design", Source configuration, MoE bullet).
 *
 * Learned mode (hash_table == NULL):
 *   z[t,e] = sum_h x[t,h] * w_router[h,e]
 *   s      = sqrt(softplus(z))
 *   ids[t] = the top_k experts by s + sel_bias[e] (sel_bias NULL = 0), in
 *            descending key order, equal keys to the lower expert id
 *   weights[t,j] = route_scale * s[ids[t,j]] / sum_j s[ids[t,j]]  (unbiased s)
 * The ids are those of the float64 z (sums of exact products, rounded only
 * in float64 additions).  T <= 256, or E not a multiple of 64, or w_router
 * not 16-byte aligned: z in float64 for every (t, e).  Otherwise z comes
 * from the bf16 matrix cores (w_router split exactly into three bf16 terms,
 * float32 sums of each 32-long k step added in float64) with a bound on its
 * error; a token whose selection the bound cannot decide gets float64 z, and
 * chosen experts whose order the bound cannot decide, or whose s is below
 * sqrt(softplus(4)), get float64 z before ordering and weighting.  The
 * remaining z carry that rounding (about 1e-6 absolute at |z| ~ 20), which
 * moves a weight by well under 1e-6 relative.
 * Hash mode (hash_table != NULL): ids[t,j] = hash_table[token_ids[t]*top_k + j]
 *   and weights = route_scale / top_k.  A token id outside [0, V) gives ids -1
 *   for that token (moe_dispatch then drops those pairs).
 *
 * x        bf16 [T, H] row-major, 16-byte aligned
 * w_router float32 [H, E] row-major (learned mode)
 * sel_bias float32 [E] or NULL
 * token_ids int32 [T], hash_table int32 [V, top_k] (hash mode)
 * ids      int32 [T, top_k] out;  weights float32 [T, top_k] out
 * ws       device workspace of at least moe_route_workspace_size(T, H, E) bytes,
 *          256-byte aligned (learned mode; may be NULL in hash mode)
 * Requirements: 1 <= top_k <= 8, top_k <= E <= 256, H a positive multiple of
 * 512 up to MOE_MAX_DIM (MOE_ESHAPE otherwise).
 */
size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E);
int moe_route(const uint16_t* x, int32_t T, int32_t H, const float* w_router, const float* sel_bias,
              const int32_t* token_ids, const int32_t* hash_table, int32_t V, int32_t E, int32_t top_k,
              float route_scale, int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream);

/*
 * Dispatch: groups the (token, slot) pairs by expert for the experts call
 * ("Model techniques map -- DeepSeek-V4-Flash", row "Shared expert": the
 * experts module takes the flattened tokens with the routed ids and weights).
 * Rows are ordered by (expert, token, slot) -- a stable counting sort -- and
 * the shared-expert group (every token, in order) comes last.
 *
 * ids       int32 [T, top_k] in
 * offsets   int32 [E + 2] out: group g (g < E routed, g = E shared) owns rows
 *           offsets[g] .. offsets[g+1]-1; offsets[E+1] = total rows
 * row_token int32 [T * (top_k + 1)] out: token of each row
 * slot_row  int32 [T, top_k + 1] out: row of pair (t, j); column top_k is the
 *           shared-expert row of t
 * Ids outside [0, E) get no row and slot_row -1 (they contribute nothing).
 * ws: at least moe_dispatch_workspace_size(T, E, top_k) bytes, 256-byte aligned.
 */
size_t moe_dispatch_workspace_size(int32_t T, int32_t E, int32_t top_k);
int moe_dispatch(const int32_t* ids, int32_t T, int32_t E, int32_t top_k, int32_t* offsets, int32_t* row_token,
                 int32_t* slot_row, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and ordering as moe_dispatch without the
 * workspace, whose contents (per-pair ranks, per-chunk counts) live instead
 * in a static device array of MOE_DISPATCH_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing; its first call on a device looks up that device's array
 * once (with the stream's device current).  A call whose scratch need
 * (moe_dispatch_workspace_size(T, E, top_k)) exceeds the array returns
 * MOE_EWORKSPACE and enqueues nothing: at E = 256 and top_k = 6 that is
 * T > 149,000 or so.  Every word of the array a call reads it writes first,
 * so the last call's contents never leak into the next; but all calls on one
 * GPU share the array, so calls that may overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.
 */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_dispatch_noalloc(const int32_t* ids, int32_t T, int32_t E, int32_t top_k, int32_t* offsets,
                         int32_t* row_token, int32_t* slot_row, void* stream);

/*
 * Expert FFN over every dispatched row ("Model techniques map --
 * DeepSeek-V4-Flash", row "SwiGLU feed-forward"; clamping also named in
 * "DeepSeek-V4-Flash export design", V3 reuse and V4 differences):
 *   g = W_gate[e] x,  u = W_up[e] x                  (float32 accumulation)
 *   h = bf16( silu(min(g, L)) * min(max(u, -L), L) )
 *   out_rows[p] = bf16( W_down[e] h )                (float32 accumulation)
 * for each row p of group e, x = x[row_token[p]].  The MXFP4 weights are
 * decoded to bf16 on the fly and fed to bf16 MFMA (or, with MOE_FFN_SPLIT_FP8
 * in experts->flags and a prefill-sized T, fed as stored to the scaled FP4
 * matrix cores); only the experts that own rows are read.  With
 * MOE_ROUTED_AFFINE2 each routed projection is computed per group as
 * s * (x . q) + b * sum(x) (the same sum, regrouped), x . q and sum(x) on bf16
 * MFMA.
 *
 * x         bf16 [T, H]; experts: descriptor (host pointer) of the device blob
 * offsets, row_token: as written by moe_dispatch for the same T, E, top_k
 * out_rows  bf16 [T * (top_k + 1), H] out, 16-byte aligned (rows past
 *           offsets[E+1] untouched); each row rounded once (to nearest even)
 *           from its float32 sum, activations in bf16 as x and h are
 * ws        at least moe_ffn_workspace_size(T, experts, top_k) bytes, 256-byte aligned
 * clamp_limit L > 0.
 */
size_t moe_ffn_workspace_size(int32_t T, const moe_experts* experts, int32_t top_k);
int moe_expert_ffn(const uint16_t* x, int32_t T, const moe_experts* experts, int32_t top_k,
                   const int32_t* offsets, const int32_t* row_token, float clamp_limit, uint16_t* out_rows,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * The same expert FFN enqueued one launch at a time, for callers that time or
 * interleave the launches: phase 0 builds the work list from offsets, phase 1
 * runs gate/up + clamped SwiGLU into the workspace (h), phase 2 runs
 * the down projection into out_rows.  Phases 0, 1, 2 issued in order on one
 * stream with identical arguments (same workspace) equal one moe_expert_ffn
 * call bit for bit.  phase -1 runs all three; any other value is MOE_EINVAL.
 */
int moe_expert_ffn_phase(const uint16_t* x, int32_t T, const moe_experts* experts, int32_t top_k,
                         const int32_t* offsets, const int32_t* row_token, float clamp_limit,
                         uint16_t* out_rows, void* ws, size_t ws_bytes, int32_t phase, void* stream);

/*
 * Weighted combine plus the shared expert ("Model techniques map --
 * DeepSeek-V4-Flash", row "Shared expert"):
 *   y[t] = bf16( sum_{j<top_k} weights[t,j] * out_rows[slot_row[t,j]]
 *                + out_rows[slot_row[t,top_k]] )
 * summed in float32 in that fixed order (the deterministic reduction the
 * techniques map lists under inference kernels).  slot_row entries of -1 are
 * skipped.
 * out_rows bf16 [rows, H]; slot_row int32 [T, top_k+1]; weights float32
 * [T, top_k]; y bf16 [T, H] out.  H a positive multiple of 8.
 */
int moe_combine(const uint16_t* out_rows, const int32_t* slot_row, const float* weights, int32_t T, int32_t H,
                int32_t top_k, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
