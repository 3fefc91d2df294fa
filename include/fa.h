/*
 * fa.h -- C ABI of the exact tiled-attention library for AMD MI355X (gfx950).
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V for every
 * (batch, head) pair, block by block with an online softmax so that the
 * N x N score and probability matrices never reach device memory, and the
 * matching backward pass that recomputes them from the stored per-row
 * log-sum-exp.  Definitions:
 *   - attention, S and P: "Overview of Flash Attention series", section
 *     Standard Attention Implementation / Forward Pass; the 1/sqrt(d) scale
 *     as in the "Transformer 入门" (Transformer primer) definitions;
 *   - online softmax and output rescaling: "FlashAttention in NeurIPS 2022"
 *     (coreui blog) section 2.1, and "Как работает FlashAttention
 *     математически" sections 3-4;
 *   - stored statistics and recomputation: "Overview of Flash Attention
 *     series", sections Tiling and Forward Pass of flashattention (the
 *     normaliser L_i), and section 5 of the aivaro.ru answer;
 *   - gradients: "Overview of Flash Attention series", section Backward Pass
 *     of flashattention (dV = P^T dO, dP = dO V^T, D_i = do_i . o_i,
 *     dS = P o (dP - D), dq_i = sum_j dS_ij k_j, dk_j = sum_i dS_ij q_i).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or copies to the host, and keeps no
 *     state between calls (calls are reentrant).
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are contiguous row-major
 *     [B, H, N, d] (d fastest) in the element type `dtype`; lse is
 *     contiguous [B, H, N] float32.  Pointers must be 16-byte aligned.
 *   - `causal` != 0 keeps key index <= query index (masked scores are -inf).
 *   - `scale` multiplies Q K^T before the softmax (1/sqrt(d) for standard
 *     attention); it must be finite and >= 0.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; results are valid once the caller synchronises the
 *     stream.  The calls enqueue kernels only (no allocation, memset, copy or
 *     synchronisation), so they can be captured into a HIP graph and
 *     replayed; make the first call of each kind outside a capture (it sets
 *     a kernel's LDS limit once per process).
 *   - Outputs must not alias inputs.
 *   - B, H or N equal to 0 describes an empty problem: the call validates the
 *     pointers it can, enqueues nothing and returns FA_OK.
 *   - Arguments are validated before any HIP call: an invalid call returns a
 *     non-zero fa_status and enqueues nothing.  FA_ERR_HIP reports a launch
 *     failure (hipGetLastError after the launch).  No C++ exception crosses
 *     this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O, dO, dQ, dK, dV.  Accumulation is always fp32. */
enum fa_dtype {
  FA_F32 = 0,  /* IEEE float32 */
  FA_BF16 = 1  /* bfloat16; outputs rounded to nearest even */
};

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL (non-empty problem) */
  FA_ERR_SHAPE = 2,     /* B, H or N negative; one head's (N + 256) * d elements exceed 2^31 - 1 bytes; or
                           B * H * ceil(N / 128) is 2^23 or more (a launch's work items must fit in 32 bits) */
  FA_ERR_HEADDIM = 3,   /* d is not 64 or 128 */
  FA_ERR_DTYPE = 4,     /* dtype is not an fa_dtype */
  FA_ERR_SCALE = 5,     /* scale is NaN, infinite or negative, or scale * log2(e) overflows float (FP8: a descale
                           factor not finite or <= 0, or scale * q_descale * k_descale * log2(e) overflows float) */
  FA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than fa_backward_workspace_size */
  FA_ERR_HIP = 7,       /* the HIP runtime reported an error at launch */
  FA_ERR_ALIGN = 8,     /* a tensor pointer is not 16-byte aligned */
  FA_ERR_MASK = 9,      /* block-sparse mask geometry invalid (see fa_forward_block_sparse) */
  FA_ERR_DROPOUT = 10,  /* dropout probability outside [0, 255/256] after rounding (see fa_forward_dropout) */
  FA_ERR_SCRATCH = 11   /* fa_backward_noalloc: the problem needs more than FA_NOALLOC_SCRATCH_BYTES of workspace */
};

/*
 * Forward pass.  Q, K, V are [B,H,N,d]; writes O [B,H,N,d] (same dtype) and
 * lse [B,H,N] (float32, lse_i = ln sum_j exp(scale * q_i . k_j) over the
 * unmasked keys j -- the log of the normaliser L_i of "Overview of Flash
 * Attention series", kept for the backward's recomputation).  Each workgroup
 * owns a tile of query rows, keeps its running row max m, row sum l and the
 * un-normalised output in registers while streaming K/V tiles through LDS
 * (the Q-outer "V2" loop order of the Transformer primer), and divides by l
 * once at the end.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, int dtype,
               void* stream);

/*
 * Block-sparse forward pass ("Overview of Flash Attention series", section
 * Block-sparse Flashattention): attention restricted by a mask that is
 * constant on blocks of block_q query rows by block_k keys.  Masked entries
 * carry no weight at all (the blocks are skipped, as the page's algorithm
 * does; its formula S o 1_M is read as excluding them, like the causal mask).
 *   block_mask: DEVICE pointer, uint8, contiguous
 *     [mask_heads][ceil(N/block_q)][ceil(N/block_k)]; non-zero keeps a block.
 *     mask_heads = 1 applies one mask to every (batch, head); mask_heads = H
 *     gives head h the mask h, shared by the batch.  Read-only.
 *   block_q: a positive multiple of 32; block_k: a positive multiple of 64.
 *   N <= 65536.  Violations return FA_ERR_MASK.
 *   causal != 0 additionally keeps key index <= query index.
 * Everything else as fa_forward.  A query row that keeps no key gets O = 0
 * and lse = -inf.  Key tiles masked out for a whole workgroup are neither
 * read from memory nor computed, so the work and the K/V traffic scale with
 * the kept fraction of blocks.
 */
int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const unsigned char* block_mask, int mask_heads, int block_q, int block_k,
                            int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Split-KV decoding ("Как работает FlashAttention математически", section 9,
 * FlashDecoding): Nq new query rows attend to Nk cached keys and values.
 *   q, o: [B, H, Nq, d] with 1 <= Nq <= 32 (Nq = 0 is an empty problem);
 *   k, v: [B, H, Nk, d] with Nk >= 1 (the cache);  lse: [B, H, Nq] float32.
 *   The queries are the LAST Nq positions of the sequence: causal != 0 lets
 *   query i see keys 0 .. Nk - Nq + i (and requires Nq <= Nk); causal = 0
 *   lets every query see all Nk keys.
 * The keys of each head are cut into num_splits chunks of 32-key tiles (0
 * picks a number that fills the GPU; more chunks than tiles are not used).
 * Each chunk's partial result goes to `workspace`, and a second kernel
 * merges them with the rule for concatenated key blocks ("Overview of Flash
 * Attention series", Tiling); with one chunk per head the outputs are
 * written directly.
 * `workspace`: a device buffer of at least
 * fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits) bytes (0 bytes, and
 * NULL allowed, when one chunk per head is used), 256-byte aligned; contents
 * on entry are ignored, on exit unspecified.  Calls that run concurrently
 * must not share a workspace.
 * Shape errors (Nq > 32, Nk < 1, causal with Nq > Nk, num_splits < 0, or
 * B * H * max(chunks, Nq) of 2^26 or more, past the grids' 32-bit work-item
 * limit) return FA_ERR_SHAPE.  Everything else as fa_forward.
 */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits);
/* The number of key chunks fa_decode uses for these sizes (0 for invalid sizes). */
int fa_decode_num_splits(int B, int H, int Nk, int num_splits);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, int causal, float scale, int dtype,
              int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace that fa_backward needs: two fp32 row statistics
 * per (batch, head, row) -- D = rowsum(dO o O) and -lse in the kernels'
 * exponent domain -- each array 256-byte aligned.  Linear in N: no N x N
 * buffer is ever used.  Returns 0 for invalid or empty shapes.
 */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass.  Inputs: Q, K, V, O, dO [B,H,N,d] and lse [B,H,N] from
 * fa_forward on the same Q, K, V, causal and scale.  Writes dQ, dK, dV
 * [B,H,N,d] (same dtype).  `workspace` is a caller-owned device buffer of at
 * least fa_backward_workspace_size(B,H,N,d) bytes, 256-byte aligned; its
 * contents on entry are ignored and on exit are unspecified.  P is
 * recomputed as exp(scale * Q K^T - lse) ("Как работает FlashAttention
 * математически" section 5).  The result is deterministic (no atomics).
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, int causal, float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse backward pass: the gradients of fa_forward_block_sparse
 * ("Overview of Flash Attention series", section Block-sparse
 * Flashattention: the backward skips the same zero blocks as the forward).
 * Inputs O and lse come from fa_forward_block_sparse with the same mask,
 * mask_heads, block_q, block_k, causal and scale; the mask arguments follow
 * the same rules (FA_ERR_MASK otherwise), everything else as fa_backward
 * (the workspace is fa_backward_workspace_size bytes).  Blocks the mask
 * removes get no gradient, and rows that keep no key get dQ = 0.  The
 * preprocess pass (D = rowsum(dO o O)) runs over every row; the dK/dV and
 * dQ passes visit only kept blocks, so their work scales with the kept
 * fraction.  Deterministic (no atomics).
 */
int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const unsigned char* block_mask, int mask_heads, int block_q, int block_k,
                             int B, int H, int N, int d, int causal, float scale, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward with 8-bit float inputs.  q, k, v: [B,H,N,d] in the OCP FP8 format
 * E4M3 (one byte per element: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, no infinities, largest finite 448), each tensor with one
 * descale factor: an element's value is its stored number times the factor
 * (finite and > 0, else FA_ERR_SCALE).  Computes
 *   O = softmax(scale * (q_descale Q)(k_descale K)^T) (v_descale V)
 * with O written in bfloat16 [B,H,N,d] and lse [B,H,N] float32 as in
 * fa_forward.  Both products run on the 8-bit matrix core (fp32
 * accumulation); the probabilities are rounded to E4M3 (nearest even) before
 * they multiply V, while the row sums use them unrounded.  FP8 is named on
 * "Как работает FlashAttention математически", section 9 (FlashAttention-3),
 * without a format; format and scaling are this library's.  Everything else
 * as fa_forward.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   float q_descale, float k_descale, float v_descale, void* stream);

/*
 * Attention with dropout on the probabilities, forward and backward
 * ("Как работает FlashAttention математически", section 5; "Overview of
 * Flash Attention series", Backward Pass: masks are regenerated, not stored):
 *   O = (P o Z) V / (1 - t/256),  P = softmax(scale * Q K^T),
 * lse that of the undropped scores.  The keep mask Z is a pure function of
 * (seed, offset, b * H + h, query, key), so the backward, called with the
 * same seed and offset, regenerates it: element (i, j) of head bh takes
 * byte 4 (i mod 4) + (j mod 4) (little-endian within the words) of the
 * counter-based generator Philox4x32-10 (Salmon et al., SC 2011) at counter
 * (j / 4, i / 4, bh, offset) with key (seed low word, seed high word), and is
 * dropped when that byte is < t.  The drop probability p_drop is quantised
 * to t / 256 with t = floor(256 p_drop + 0.5) in float32; t outside [0, 255]
 * (or a non-finite p_drop) returns FA_ERR_DROPOUT.  t = 0 is attention
 * without dropout.  The backward uses
 *   dV = (P o Z)^T dO / (1 - t/256),  dS = P o (dP o Z / (1 - t/256) - D),
 * with D_i = do_i . o_i as without dropout.  Everything else as fa_forward
 * and fa_backward.
 */
int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale, int dtype,
                       float p_drop, unsigned long long seed, unsigned offset, void* stream);
int fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        float p_drop, unsigned long long seed, unsigned offset,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages that fa_backward enqueues, in order, for callers that
 * schedule or time them separately.  Same tensors, layout, scale and
 * workspace as fa_backward; fa_backward_preprocess fills the workspace and
 * the other two read it, in either order, on the same stream.
 *   fa_backward_preprocess: D_i = do_i . o_i (fp32, the row term of the
 *     softmax Jacobian, "Overview of Flash Attention series", Backward Pass)
 *     and -lse_i into the workspace.
 *   fa_backward_dkdv: recompute S and P key block by key block and write
 *     dK = scale * dS^T Q and dV = P^T dO.
 *   fa_backward_dq: recompute them query block by query block and write
 *     dQ = scale * dS K.
 */
int fa_backward_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N,
                           int d, int dtype, void* workspace, size_t workspace_bytes, void* stream);
int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                     void* dv, int B, int H, int N, int d, int causal, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);
int fa_backward_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                   int B, int H, int N, int d, int causal, float scale, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_backward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * validation, kernels and results as fa_backward, bit for bit.  The workspace
 * lives in a device array of FA_NOALLOC_SCRATCH_BYTES inside the library,
 * which each GPU the library runs on holds until the process ends; the call
 * itself allocates and frees nothing.  Problems whose
 * fa_backward_workspace_size exceeds FA_NOALLOC_SCRATCH_BYTES (B*H*N above
 * about two million rows) return FA_ERR_SCRATCH.  All calls on one GPU share
 * that GPU's array: calls that overlap in time on one GPU (on different
 * streams or host threads) race and must be serialised by the caller.  The
 * first call on each device looks the array up (hipGetSymbolAddress); make it
 * outside a graph capture.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale, int dtype, void* stream);

/* Static English description of an fa_status value (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
