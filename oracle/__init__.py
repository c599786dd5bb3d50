"""CPU oracle for paged decode attention and the per-step K/V append.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check and the bench's CPU-baseline leg use it.  It
shares no code with the HIP library: it is plain numpy in float64, written
from the definitions on the source pages, and deliberately slow and obvious.

Pages cited (by title and section):
  [P1] "KV Cache from first principles" (ldpk.cn/news/58971): 2.1 scaled
       dot-product attention; 2.2 decode attends over cached K/V; 2.3 append
       at the current length; 3.1 bytes per token; 3.2 worked model table;
       4.3 paging; 5.1 GQA/MQA; 5.3 sliding window and attention sinks.
  [P2] "Large-model inference KV Cache memory optimisation: from PagedAttention
       to AI memory systems" (wmrh.cn/news/79784): 1.1 KV size formula and the
       13B example; 2.2 fixed-size blocks and block tables; 3.1-3.2 sharing.
  [P3] "Training and inference memory ledger" (pptc.cn/news/143802): 3.2 KV
       capacity formula and the 7B example; 3.3 GQA groups; 4.1 7B budget.
  [P4] "Why does KV Cache eat GPU memory? What does PagedAttention solve?"
       (yfxerp.com/news/121119): the per-request byte formula and 32L/8KV
       example; decode reads history then appends; FP8 KV.
  [P5] "The KV Cache memory ledger: PagedAttention and continuous batching"
       (gcssc.sfwss.com/posts/kv-cache-budget.html): 1 bytes per token (70B);
       2 GQA table; 4 block table; 4 prefix sharing; 7 quantized
       KV with per-head scales; sink tokens kept out of coarse quantisation.

Readings taken where the pages are silent (each is also a test):
  * cache memory order is [num_blocks, kv_heads, block_size, head_dim];
  * query head i uses KV head i // g (contiguous groups of g = Hq / Hkv);
  * the new token is appended first and attended to (lengths count it);
  * a sequence of length 0 yields a zero output row;
  * fp8 is OCP e4m3fn (bias 7, max 448, no inf, NaN = S.1111.111), int8 is
    symmetric (codes -127..127), and a stored value is code_value * scale
    with one fp32 scale per (block, head), times an optional per-(head,
    channel) factor for K.

Every function here is pinned by a -m "not gpu" test against something other
than itself (a library routine, a closed form, an invariant, or a number the
pages print); none is "parity unpinned".
"""

from .fp8_e4m3 import decode_e4m3fn, encode_e4m3fn_rne, E4M3_MAX, E4M3_NAN_CODES
from .values import stored_to_f64
from .paged_attention import page_of, gather_sequence, paged_decode_attention, attended_positions
from .kv_append import kv_append_bits, kv_append_fp8, kv_append_int8, kv_append_quant
from .kv_bytes import kv_bytes_per_token, kv_bytes

__all__ = [
    "decode_e4m3fn",
    "encode_e4m3fn_rne",
    "E4M3_MAX",
    "E4M3_NAN_CODES",
    "stored_to_f64",
    "page_of",
    "gather_sequence",
    "paged_decode_attention",
    "attended_positions",
    "kv_append_bits",
    "kv_append_fp8",
    "kv_append_int8",
    "kv_append_quant",
    "kv_bytes_per_token",
    "kv_bytes",
]
