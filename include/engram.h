/*
 * engram.h - C ABI of libengram, the MI355X (gfx950) Engram forward path.
 *
 * Engram is a conditional-memory layer: each position hashes its recent
 * compressed tokens into a large static table, gathers the selected rows,
 * projects them to keys and a value, and gates the value into the hidden
 * state. Sources (web pages on Engram):
 *   [zLLM]    zhuai.tech, "DeepSeek V4.1 Flash 的 Engram：让知识不必每次重新算"
 *   [Storage] lqnn.cn, "3.84 亿行 Embedding 的存法大揭秘"
 *   [vLLM]    data-sketchers.com wiki, "Engram: n-gram 조회를 통한 조건부 메모리"
 *
 * Conventions for every entry point:
 *  - Array pointers are DEVICE pointers owned by the caller. The library never
 *    allocates or frees memory the caller sees, keeps no state between calls
 *    (apart from engram_forward_noalloc's device array, see there) and never
 *    synchronises the host with the device.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    at once. Calls are thread-safe (engram_forward_noalloc calls that overlap
 *    on one GPU race on its array).
 *  - BF16 values travel as uint16_t bit patterns.
 *  - Shapes, pointers, alignment and parameter tables are checked on the host
 *    before anything is launched; a failed check returns ENGRAM_EINVAL and
 *    launches nothing (engram_last_error() says which check failed).
 *  - Violations the host cannot see without reading device memory (a token
 *    id >= map_len, a map value >= vocab_c, a row index >= n_rows,
 *    cu_seqlens that are not a non-decreasing list from 0 to T) never cause
 *    an out-of-bounds access. If `err_flags` is non-NULL the kernels OR the
 *    ENGRAM_ERR_* bits into it; the affected outputs are then unspecified
 *    but written in bounds.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_ABI_VERSION 3

/* Status codes returned by every entry point. */
#define ENGRAM_OK            0
#define ENGRAM_EINVAL       (-1)  /* host-side shape, pointer, alignment or parameter check failed */
#define ENGRAM_EHIP         (-2)  /* a HIP launch or runtime call failed */
#define ENGRAM_EUNSUPPORTED (-3)  /* valid request this library does not handle (e.g. not gfx950) */

/* Device-side error bits (ORed into *err_flags when err_flags != NULL). */
#define ENGRAM_ERR_TOKEN_RANGE 0x1u  /* a non-DEAD token id >= map_len (hashed as pad_cid) */
#define ENGRAM_ERR_MAP_RANGE   0x2u  /* a token map value >= vocab_c */
#define ENGRAM_ERR_ROW_RANGE   0x4u  /* a row index >= n_rows that is not ENGRAM_DEAD_IDX (row written as 0) */
#define ENGRAM_ERR_SEQLENS     0x8u  /* cu_seqlens not non-decreasing from 0 to T */

/* Fixed geometry: 2/3/4-grams x 8 heads = 24 rows of 256 values per token
 * per layer, 3 x 8 x 256 = 6,144 memory values ([zLLM] 把知识变成可寻址的向量). */
#define ENGRAM_BUCKETS        24
#define ENGRAM_HEADS_PER_ORDER 8
#define ENGRAM_ROW            256
#define ENGRAM_SCALES_PER_ROW 8      /* one E8M0 scale per 32 values ([zLLM] 第二步) */
#define ENGRAM_MEM            6144
#define ENGRAM_HIST           3      /* history slots: the three most recent compressed ids */

#define ENGRAM_DEAD_TOKEN 0xFFFFFFFFu /* token value of an image (DEAD) position ([zLLM] 第四步) */
#define ENGRAM_DEAD_IDX   0xFFFFFFFFu /* row index written for a DEAD position */

/* One layer's hash parameters ([zLLM] 第一步: per-layer multipliers, prime
 * buckets and bucket offsets expanded to static tables; [vLLM] How it works:
 * each (order, head) pair indexes its own prime-sized bucket range).
 * Bucket j = (n-2)*8 + head has order n = 2 + j/8. Passed by pointer to a
 * HOST struct; it is copied into the kernel arguments. */
typedef struct {
  uint64_t mult[ENGRAM_BUCKETS][4]; /* multiplier of window slot k (k < n) for bucket j */
  uint32_t prime[ENGRAM_BUCKETS];   /* bucket sizes: distinct primes */
  uint64_t offset[ENGRAM_BUCKETS];  /* offset[0] = 0, offset[j+1] = offset[j] + prime[j] */
  uint64_t n_rows;                  /* offset[23] + prime[23]; must be < 0xFFFFFFFF */
  uint32_t vocab_c;                 /* compressed vocabulary size */
  uint32_t pad_cid;                 /* id hashed for history slots before the start or behind a DEAD */
} engram_hash_params;

/* Number of hipEvent_t handles engram_forward records when given events. */
#define ENGRAM_STAGE_EVENTS 5

/* ---------------------------------------------------------------- status */

/* Static text for a status code. Never NULL. */
const char* engram_status_string(int status);

/* Detail of the last ENGRAM_EINVAL / ENGRAM_EHIP returned on this thread
 * (empty string if none). Valid until the next call on this thread. */
const char* engram_last_error(void);

/* ENGRAM_ABI_VERSION of the built library. */
int engram_abi_version(void);

/* ---------------------------------------------------------------- parameters */

/* Pure host check of one layer's parameters against its token map
 * ([vLLM] How it works: a compressed-vocabulary mismatch must fail at
 * start-up). Checks: every prime[j] is prime and the 24 are distinct; the
 * offsets are the prefix sums of the primes, so bucket ranges are disjoint
 * and tile [0, n_rows); n_rows < 0xFFFFFFFF; vocab_c >= 1; pad_cid <
 * vocab_c; every token_map_host[i] < vocab_c. token_map_host is a HOST
 * array of map_len entries (may be NULL when map_len == 0). No GPU needed. */
int engram_check_params(const engram_hash_params* params,
                        const uint32_t* token_map_host, uint32_t map_len);

/* ---------------------------------------------------------------- history
 * Per-sequence hash history: hist[S][3] uint32 compressed ids, hist[s][0] the
 * most recent. Each token enters the history exactly once per step, after
 * every Engram layer of that step has read it; sessions share weights but
 * not history; fork copies, reset clears ([zLLM] 第四步). */

/* hist[s][*] = pad_cid for s < S. */
int engram_history_reset(uint32_t* hist, int32_t S, uint32_t pad_cid, hipStream_t stream);

/* dst[s][*] = src[s][*] for s < S (a forked session's own copy). */
int engram_history_fork(uint32_t* dst, const uint32_t* src, int32_t S, hipStream_t stream);

/* Append one step's tokens. Sequence s owns tokens [cu_seqlens[s],
 * cu_seqlens[s+1]) of tok[T] (cu_seqlens: int32[S+1], 0 = cu[0] <= ... <=
 * cu[S] = T; empty sequences allowed). For each token in order: a DEAD
 * token resets the history to pad_cid; any other token t pushes
 * map[t] (hist becomes [map[t], h0, h1]). In place; sequences independent. */
int engram_history_append(uint32_t* hist, const uint32_t* tok, const int32_t* cu_seqlens,
                          int32_t S, int64_t T, const uint32_t* token_map, uint32_t map_len,
                          uint32_t pad_cid, uint32_t* err_flags, hipStream_t stream);

/* ---------------------------------------------------------------- stages */

/* Hash (retrieval, first half): idx[T][24] uint32 row numbers.
 * Window of a text token t: [c_t, h0, h1, h2] where c_t = token_map[tok[t]]
 * and h is the history just before t within its sequence (the read-only
 * `hist` before the first token; pad_cid behind a DEAD) ([zLLM] 第一步).
 * Bucket j of order n: x = XOR_{k<n} (w_k * mult[j][k] mod 2^64),
 * idx[t][j] = offset[j] + x mod prime[j] ([vLLM] How it works, multi-head
 * hashing). DEAD tokens get ENGRAM_DEAD_IDX in all 24 slots. `hist` is not
 * modified (call engram_history_append once per step, after all layers).
 * Alignment: tok, idx, hist, cu_seqlens 4-byte. T may be 0. */
int engram_hash(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                const engram_hash_params* params, uint32_t* idx,
                uint32_t* err_flags, hipStream_t stream);

/* Gather + decode (retrieval, second half): mem[T][6144] BF16.
 * mem[t][j*256 + c] = E4M3(codes[r][c]) * 2^(scales[r][c/32] - 127) with
 * r = idx[t][j], rounded to BF16 (nearest even; exact for every finite value
 * with |v| >= 2^-133); NaN (code S.1111.111 or scale 255) gives
 * sign(code)|0x7FC0 ([zLLM] 第二步: read only the selected rows and their
 * scales; [Storage]: FP8 E4M3 with UE8M0 group-32 scales decoded to BF16).
 * ENGRAM_DEAD_IDX rows give zeros. codes: uint8[n_rows][256] (16-byte
 * aligned), scales: uint8[n_rows][8] (8-byte aligned), mem 16-byte aligned.
 * The table (codes and scales, here and in engram_forward) may be device
 * memory or pinned host memory that is mapped into the device's address
 * space at its host address (hipHostMalloc); the rows then cross the host
 * link, as with the pages' host-resident tables ([vLLM] CPU offload). Other
 * host memory must not be passed: the kernels read it directly. */
int engram_gather_decode(const uint32_t* idx, int64_t T, const uint8_t* codes,
                         const uint8_t* scales, uint64_t n_rows, uint16_t* mem,
                         uint32_t* err_flags, hipStream_t stream);

/* wkv projection: kv[T][(hc+1)*H] = mem[T][6144] . wkv[(hc+1)*H][6144]^T,
 * BF16 inputs, FP32 accumulation, BF16 (nearest even) output. Columns
 * [b*H, (b+1)*H) of kv are key b (b < hc); [hc*H, (hc+1)*H) the shared value
 * ([zLLM] 第二步: wkv 25,600 x 6,144 BF16; [Storage] 旋转合同: the last 5,120
 * rows are V; [vLLM] How it works: one key per hyper-connection branch and
 * one shared value). Requires H % 64 == 0, 1 <= hc <= 8, 16-byte aligned
 * pointers. T may be 0.
 * wkv_packed: NULL, or the same weights in the decode layout written by
 * engram_pack_wkv (caller-owned, read-only here). Batches of at most 256
 * tokens then stream wkv_packed instead of wkv; the results are
 * bit-identical. Larger batches always read wkv. */
int engram_project(const uint16_t* mem, int64_t T, const uint16_t* wkv, const uint16_t* wkv_packed,
                   int32_t H, int32_t hc, uint16_t* kv, hipStream_t stream);

/* Writes wkv[(hc+1)*H][6144] in the decode layout into wkv_packed (caller-
 * owned device memory of the same size, 16-byte aligned, not overlapping
 * wkv); once per weight load, enqueued on `stream`. A decode step reads all
 * of wkv for a few tokens ([zLLM] AVX-512 BF16: decode gets no reuse of a
 * weight load; the pages' CPU kernels read wkv in a packed block layout of
 * their own), so it is bound by how fast wkv streams: in this layout each
 * load instruction of the decode kernel reads 1 KB that is contiguous,
 * where rows of wkv give it 64-byte pieces of 16 rows 12 KB apart.
 * Layout, with N = (hc+1)*H and G = min(112, max(16, ceil(N / 256))): rows
 * form groups of G (the last may be shorter), each cut in tiles of 16 rows
 * (the group's last tile may be shorter, r rows in all). Value k of row n0+i
 * of a tile starting at row n0, with k = 64s + 16g + 8j + e (s < 96, g < 4,
 * j < 2, e < 8), sits at index n0*6144 + (((2s + j)*4 + g)*r + i)*8 + e.
 * Returns ENGRAM_EINVAL for bad H/hc, NULL, misaligned or overlapping
 * buffers. */
int engram_pack_wkv(const uint16_t* wkv, int32_t H, int32_t hc, uint16_t* wkv_packed,
                    hipStream_t stream);

/* Context gate + residual, in place on hidden[T][hc][H] BF16.
 * For each non-DEAD token and branch b (DEAD = tok[t] == ENGRAM_DEAD_TOKEN,
 * tok may be NULL for no DEAD positions):
 *   r_h = 1/sqrt(mean(h_b^2) + eps), r_k = 1/sqrt(mean(k_b^2) + eps)
 *   dot = dot_scale * r_h * r_k * sum_i h_b[i] * k_b[i] * wqk[b][i]
 *   g   = sigmoid(copysign(sqrt(max(|dot|, 1e-6)), dot))
 *   h_b = bf16(h_b + g * v)
 * ([zLLM] 第三步; [vLLM] How it works, fusion). DEAD rows are left
 * bit-identical and get g = 0 ([zLLM] 第四步: image rows skip the gate).
 * wqk: float32[hc][H] (premultiplied q and k norm weights). gate_out:
 * float32[T][hc] or NULL. Requires H % 64 == 0, 1 <= hc <= 8, 16-byte
 * aligned hidden/kv/wqk. */
int engram_gate(uint16_t* hidden, const uint16_t* kv, const float* wqk, const uint32_t* tok,
                int64_t T, int32_t H, int32_t hc, float eps, float dot_scale,
                float* gate_out, hipStream_t stream);

/* ---------------------------------------------------------------- whole layer */

/* Workspace bytes engram_forward (and engram_precompute) needs for T
 * tokens. Layout, each section 256-byte aligned: idx uint32[T][24] | slot
 * uint32[T] | live count uint32 and one uint32 per 4,096 positions | mem
 * bf16[T][6144] | kv bf16[T][(hc+1)*H] (at least T*24*264 bytes: rows staged
 * from a host table sit there until they are decoded) | live positions
 * uint32[T] (position of each packed row, for batches above the small-batch
 * limits). */
size_t engram_forward_workspace(int64_t T, int32_t H, int32_t hc);

/* engram_precompute flag: copy the selected rows and scales into the
 * workspace first (16-byte loads, many rows in flight), then decode them
 * from device memory; for tables in pinned host memory ([vLLM] CPU offload:
 * host-resident tables whose rows are fetched ahead of use). Without it the
 * decode reads the table in place. The results are the same either way. */
#define ENGRAM_PRECOMPUTE_STAGE_ROWS 0x1u

/* The half of one Engram layer that does not read the hidden state:
 * engram_hash -> engram_gather_decode -> engram_project, into `ws`
 * (caller-owned device memory of at least engram_forward_workspace(T, H, hc)
 * bytes, 256-byte aligned). Only the gate needs the layer's input hidden
 * state, so this can run ahead of the layer, e.g. on a side stream while the
 * layers before it run ([zLLM] 提前投影: the projection is issued before the
 * layer is reached and only the gate waits for the hidden state; [FlagOS]
 * 4.1: the lookup is prefetched and overlapped with compute).
 * Arguments mean what they mean in the stage calls; every host check runs
 * before anything is enqueued; the library allocates nothing. `hist` is read
 * only and must hold the history before this step (call
 * engram_history_append once per step, after every layer's precompute has
 * been enqueued on, or ordered before, the append's stream).
 * flags: 0 or ENGRAM_PRECOMPUTE_STAGE_ROWS.
 * For T <= 1024 tokens in S <= 1024 sequences, mem/kv row t belongs to
 * position t (hash, gather and decode run as one kernel unless rows are
 * staged). Larger batches decode and project only the live (non-DEAD)
 * positions, packed in position order: slot[t] is the row of position t
 * or ENGRAM_DEAD_IDX, and the live count is read on the device.
 * The workspace then holds everything engram_gate_precomputed reads. */
int engram_precompute(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                      const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                      const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                      const uint16_t* wkv, const uint16_t* wkv_packed, int32_t H, int32_t hc,
                      uint32_t flags, void* ws, size_t ws_bytes, uint32_t* err_flags,
                      hipStream_t stream);

/* A layer's table kept as one allocation per bucket: bucket j's rows
 * offset[j] .. offset[j] + prime[j] - 1 (engram_hash_params) are the
 * uint8[prime[j]][256] codes at codes[j] and the uint8[prime[j]][8] scales at
 * scales[j] (16- and 8-byte aligned; device memory or pinned host memory
 * mapped at its host address, as for the one-allocation table). For tables
 * in pinned host memory, where one allocation of a full-size table (98.3 GB
 * of codes) may be refused ([vLLM] CPU offload: tables stay in host
 * memory and HBM holds the KV cache instead). */
typedef struct {
  const uint8_t* codes[ENGRAM_BUCKETS];
  const uint8_t* scales[ENGRAM_BUCKETS];
} engram_bucket_table;

/* engram_precompute with the table given per bucket (engram_bucket_table):
 * the same work, results and checks; a row is read from its bucket's
 * allocation. */
int engram_precompute_buckets(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                              const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                              const engram_hash_params* params, const engram_bucket_table* table,
                              const uint16_t* wkv, const uint16_t* wkv_packed, int32_t H, int32_t hc,
                              uint32_t flags, void* ws, size_t ws_bytes, uint32_t* err_flags,
                              hipStream_t stream);

/* The gate at layer entry ([zLLM] 提前投影: only the gate reads the layer's
 * hidden state): engram_gate on hidden[T][hc][H] with the keys and value
 * that engram_precompute left in `ws` for the same tok, S, T, H and hc
 * (anything else is undefined: the workspace layout depends on T and S).
 * DEAD positions pass through bit-identical with gate 0. The precompute must
 * be complete or ordered before this call on `stream` (an event wait when it
 * ran on another stream). Requires tok (the DEAD mask) for T > 0. */
int engram_gate_precomputed(uint16_t* hidden, const void* ws, size_t ws_bytes, const uint32_t* tok,
                            int32_t S, int64_t T, const float* wqk, int32_t H, int32_t hc,
                            float eps, float dot_scale, float* gate_out, hipStream_t stream);

/* One Engram layer: engram_precompute (flags 0) followed by
 * engram_gate_precomputed, enqueued on one stream with intermediates in `ws`
 * (caller-owned device memory of at least engram_forward_workspace(T, H, hc)
 * bytes, 256-byte aligned). Arguments mean what they mean in the stage
 * calls, and every stage's host checks run before anything is enqueued (an
 * ENGRAM_EINVAL return leaves the stream untouched).
 * Per step: call once per layer with that layer's params/table/wkv/wqk and
 * hidden, all reading the same `hist`, then engram_history_append once.
 * wkv_packed (NULL or engram_pack_wkv's output for this wkv) is passed on to
 * the projection, which reads it for batches of at most 256 tokens.
 * For T <= 1024 tokens in S <= 1024 sequences (decode steps) hashing,
 * gathering and decoding run as one kernel, since both steps are chains of
 * dependent loads at that size; idx, mem and err_flags are bit-identical to
 * the two separate calls, and mem/kv row t belongs to position t.
 * Larger batches decode and project only the live (non-DEAD) positions: a
 * DEAD position passes through the gate untouched, so its k/v are never
 * read ([zLLM] 第四步: image rows skip the gate). slot[t] is then the mem/kv
 * row of position t (rows packed in position order) or ENGRAM_DEAD_IDX, and
 * the live count is read on the device (no host synchronisation). Hidden
 * states and gates are the same either way.
 * stage_events: NULL, or ENGRAM_STAGE_EVENTS hipEvent_t created by the caller,
 * recorded before hashing, after hashing, after gather+decode, after the
 * projection and after the gate (with the single hash + gather kernel, the
 * second and third are both recorded after it). */
int engram_forward(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                   const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                   const engram_hash_params* params, const uint8_t* codes, const uint8_t* scales,
                   const uint16_t* wkv, const uint16_t* wkv_packed, const float* wqk,
                   uint16_t* hidden, int32_t H, int32_t hc, float eps, float dot_scale, void* ws,
                   size_t ws_bytes, float* gate_out, uint32_t* err_flags,
                   hipEvent_t* stage_events, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): engram_forward
 * with the workspace taken from a device array of
 * ENGRAM_NOALLOC_WORKSPACE_BYTES that the library holds on each GPU it runs
 * on, until the process ends. Same arguments and results as engram_forward
 * without ws, ws_bytes and stage_events. Batches whose
 * engram_forward_workspace(T, H, hc) exceeds the array (above 1,055
 * tokens at H = 5120, hc = 4) are rejected with ENGRAM_EINVAL before any launch. The
 * call allocates nothing; the first call on a device looks up the array's
 * address there. Every call on one GPU uses the same array: calls that
 * overlap on one GPU (two streams, two threads) race, so order them. */
#define ENGRAM_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int engram_forward_noalloc(const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T,
                           const uint32_t* hist, const uint32_t* token_map, uint32_t map_len,
                           const engram_hash_params* params, const uint8_t* codes,
                           const uint8_t* scales, const uint16_t* wkv, const uint16_t* wkv_packed,
                           const float* wqk, uint16_t* hidden, int32_t H, int32_t hc, float eps,
                           float dot_scale, float* gate_out, uint32_t* err_flags,
                           hipStream_t stream);

/* ---------------------------------------------------------------- synthetic tables */

/* Writes rows [row_begin, row_begin + n_rows) of a closed-form synthetic
 * MXFP8 table, for benchmarks and tests (not part of the Engram method):
 *   codes[r][c]  = F[hi32(splitmix64(key_data + r*256 + c)) mod 254]
 *   scales[r][q] = 119 + hi32(splitmix64(key_scale + r*8 + q)) mod 9
 * where F lists the 254 non-NaN E4M3 codes in ascending order and
 * splitmix64(x) is the first output of a SplitMix64 generator (Steele, Lea
 * and Flood, 2014) whose state is x. `codes` and `scales` point at row
 * row_begin (16- and 8-byte aligned), in device memory or in pinned host
 * memory mapped at its host address; anything else is rejected with
 * ENGRAM_EINVAL before the launch. */
int engram_gen_table(uint8_t* codes, uint8_t* scales, uint64_t row_begin, uint64_t n_rows,
                     uint64_t key_data, uint64_t key_scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
