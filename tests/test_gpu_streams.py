"""Calls on different streams are independent (GPU).

The library keeps no device state between calls and allocates nothing: two
handles driven on two streams at once, each with its own workspace and
outputs, must give exactly what each gives alone. The decode kernels are
persistent (one workgroup per CU), so concurrent launches also share the
device's compute units; results must not depend on that either. All streams
are at the default priority.
"""

import pytest
import torch

import oracle
from gpu_helpers import compare, decoder_for, to_device
from workloads import make_config_case

pytestmark = pytest.mark.gpu


def _setup(name, batch, splits):
    case = make_config_case(name, batch=batch, poison=True)
    dev = to_device(case)
    dec = decoder_for(case)
    ws = dec.alloc_workspace(case.batch, splits)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
    args = dec.make_args(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                         dev["context_lens"], out, softmax_scale=case.scale, lse=lse,
                         num_splits=splits, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                         scratch_k=dev["scratch_k"], scratch_v=dev["scratch_v"])
    # The argument struct holds raw pointers: the input tensors must stay alive.
    return dec, args, ws, out, lse, (dev, case)


def test_two_streams_at_once_match_each_alone():
    jobs = [_setup("fp8_mqa_d256", 8, 0), _setup("diffusion_multitoken", 4, 3),
            _setup("llama3_8b_decode", 6, 2)]
    # Each alone, on the current stream.
    alone = []
    for dec, args, ws, out, lse, (_, case) in jobs:
        dec.launch(args, ws)
        torch.cuda.synchronize()
        O, L = oracle.run_case(case)
        compare(out, lse, O, L, "fp8" if case.kv_dtype == "fp8" else "dense", what="alone")
        alone.append((out.clone(), lse.clone()))
    streams = [torch.cuda.Stream() for _ in jobs]
    for rep in range(5):
        for _, _, _, out, lse, _ in jobs:
            out.fill_(3.0)
            lse.fill_(3.0)
        torch.cuda.synchronize()
        # Interleaved launches, no synchronisation between the streams.
        for k in range(3):
            for (dec, args, ws, _, _, _), s in zip(jobs, streams):
                dec.launch(args, ws, stream=s.cuda_stream)
        torch.cuda.synchronize()
        for i, (_, _, _, out, lse, _) in enumerate(jobs):
            assert torch.equal(out, alone[i][0]) and torch.equal(lse, alone[i][1]), (rep, i)
    for dec, *_ in jobs:
        dec.close()


def test_argument_struct_keeps_its_tensors_alive():
    """make_args returns raw device pointers; the struct must keep the input
    tensors alive on its own, so a caller that drops them and allocates
    again still launches on the right data."""
    def build():
        case = make_config_case("llama3_8b_decode", batch=4, poison=True)
        dev = to_device(case)
        dec = decoder_for(case)
        ws = dec.alloc_workspace(case.batch, 2)
        out = torch.empty_like(dev["q"])
        lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
        args = dec.make_args(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                             dev["context_lens"], out, softmax_scale=case.scale, lse=lse,
                             num_splits=2)
        return dec, args, ws, out, lse, case   # the input tensors are not returned

    dec, args, ws, out, lse, case = build()
    # Freed blocks would be handed out again here and overwritten.
    junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(64)]
    torch.cuda.synchronize()
    dec.launch(args, ws)
    torch.cuda.synchronize()
    O, L = oracle.run_case(case)
    compare(out, lse, O, L, "dense", what="after the caller dropped its inputs")
    del junk
    dec.close()
